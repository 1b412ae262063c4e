// Block-sparse exact softmax attention on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// The attention half of Sol-Attn: every query row of block i attends, with exact
// softmax, to the tokens of the key blocks selected for block i ("Videomodel
// MiniMax-H3 rendert sneller dan afspelen", section "Waar de snelheidswinst
// vandaan komt").  d = 128 and 128-token blocks.
//
// Work unit: one workgroup = one query block (128 rows) of one (b,h); 8 waves
// (two per SIMD).  Wave w owns query rows 32*(w%4)..+31 and key half kh = w/4
// (keys 64*kh..64*kh+63 of every tile).  Each wave keeps its own running max,
// sum and O over its key half; the two halves are merged once at the end
// (exact: O = sum_h 2^(m_h-m) O_h / sum_h 2^(m_h-m) l_h).  Every unit processes
// exactly topk key tiles, so units are equally expensive.
//
// Per key tile j (128 keys x 128 dims, K and V), per wave:
//   S^T = K_j Q^T      16 MFMA 32x32x16: A = K rows from LDS (16-byte reads),
//                      B = Q^T held in registers for the whole unit.  Computing
//                      S transposed puts the keys of one query in the registers
//                      of one lane pair (l, l^32), so the row max is an
//                      in-register reduction plus one cross-half exchange.
//   online softmax     in the log2 domain: t = s*scale*log2(e), m = running max,
//                      p = 2^(t-m) (v_exp_f32), l += sum p, O *= 2^(m_old-m)
//                      (skipped when no running max of the wave moved).
//   O^T += V_j^T P^T   16 MFMA 32x32x16: the S^T accumulator layout already is
//                      the B-operand layout of P^T (after bf16 rounding) for a
//                      fixed permutation of the 16 keys of each k-step; the A
//                      operand V^T is read with ds_read_b64_tr_b16, whose
//                      16-lane transpose delivers 4 consecutive keys of one
//                      column per lane, in the same key permutation.
//
// Pipelining: K and V tiles are double-buffered in LDS (4 x 32 KiB).  At the top
// of iteration t the direct-to-LDS copies of K_{t+2} and V_{t+1} are issued into
// the buffers freed by iteration t-1; the barrier closing iteration t waits for
// them.  S for tile t+1 is computed in the same iteration as the softmax and PV
// of tile t.  The two key-half waves that
// share a SIMD run the S product and the softmax in opposite order, so one
// wave's softmax (VALU, exp) overlaps the other's matrix-core work.
//
// LDS layout of a 128x128 bf16 tile: row r = 256 bytes = 16 chunks of 16 bytes;
// logical chunk c lives at physical chunk c ^ swz(r), swz(r) = 4*(r%4) + (r/4)%4.
// This makes both the 16-lane groups of 16-byte K reads (16 consecutive rows,
// same chunk) and the 32-lane groups of 8-byte transpose reads (4 consecutive
// rows x 4 consecutive chunks) hit distinct banks.
//
// Work order: workgroups are dispatched to the 8 XCDs round-robin; workgroup w
// runs on XCD w%8, and XCD x is given a contiguous range of query blocks of the
// same head as every other XCD at that moment.  All XCDs thus stream the same
// head's K/V (kept in the shared last-level cache), while each XCD's L2 serves
// the overlapping selections of its neighbouring query blocks.
#include "launchers.h"

namespace sol_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 128;
constexpr int kD = 128;
constexpr int kThreads = 512;
constexpr int kTileBytes = kBlock * kD * 2;   // 32 KiB
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.0f;   // log2 units: probabilities stay <= 256
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int lds_off(int r, int c) { return r * 256 + ((c ^ swz(r)) << 4); }

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 ds_read_tr(const unsigned char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((__attribute__((address_space(3))) unsigned char*)(base) + off));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (round to nearest even): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Global -> LDS tile copy with the gfx950 direct-to-LDS load (no register staging).
// One wave instruction writes 64 lanes x 16 bytes = 1 KiB of LDS contiguously
// (= 4 tile rows).  Lane l of segment s fills physical chunk l%16 of row
// 4s + l/16, so it fetches the logical chunk that the swizzle places there; the
// 16 lanes of a row still read that row's 256 contiguous bytes.  Wave w copies
// segments w, w+8, w+16, w+24.  Completion is awaited by the next barrier.
// Buffer resource of one head's K or V (raw, byte-addressed, range-checked: rows past
// the end of the head -- the missing rows of a short last block -- read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const unsigned char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ void tile_dma(unsigned char* lds, __amdgpu_buffer_rsrc_t r, int off, int wave,
                                         int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int seg = wave + 8 * i;
    const int row = 4 * seg + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds + seg * 1024), 16,
                                             off + row * 256 + c * 16, 0, 0, 0);
  }
}

// Scores of keys past the end of the sequence (a short last key block) -> -inf.
// s[mb][r] holds key key0 + 32mb + 8(r/4) + 4h + r%4 of the tile; `valid` keys exist.
__device__ __forceinline__ void mask_missing_keys(f32x16 (&s)[2], int key0, int h, int valid) {
  int lim = valid - key0 - 4 * h;   // key offsets 32mb + 8(r/4) + r%4 from here on are missing
  asm volatile("" : "+v"(lim));    // computed here, not hoisted as one value per register
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[mb][r] = 32 * mb + 8 * (r >> 2) + (r & 3) >= lim ? -INFINITY : s[mb][r];
}

// S^T (64 keys of this wave's half x 32 queries) = K_half . Q^T.
__device__ __forceinline__ void compute_st(f32x16 (&s)[2], const unsigned char* kt, int key0,
                                           const bf16x8 (&qf)[8], int n, int h) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    s[mb] = f32x16{};
    const int row = key0 + 32 * mb + n;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + lds_off(row, 2 * ks + h));
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0, 0);
    }
  }
  // keep at most two operand reads ahead of the matrix core (bounds register use)
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
  for (int i = 0; i < 14; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
}

__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const unsigned char* __restrict__ q, const unsigned char* __restrict__ k,
    const unsigned char* __restrict__ v, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ qblock_order, int BH, int L,
    int n_blocks, int topk, int per_xcd, float scale_log2, unsigned char* __restrict__ out,
    float* __restrict__ lse) {
  // Four separate LDS arrays (not one): the compiler can then prove that reads of
  // one buffer never alias the in-flight direct-to-LDS copies into another, and
  // does not insert a wait for those copies in the middle of the iteration.
  __shared__ __attribute__((aligned(16))) unsigned char k0s[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char k1s[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v0s[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v1s[kTileBytes];
  auto kbuf = [&](int p) { return p ? k1s : k0s; };
  auto vbuf = [&](int p) { return p ? v1s : v0s; };

  // ---- work mapping (XCD-aware, head-major across the whole chip)
  const int wg = blockIdx.x;
  const int xcd = wg % kXcds;
  const int slot = wg / kXcds;
  const int bh = slot / per_xcd;
  const int pos = xcd * per_xcd + slot % per_xcd;
  if (bh >= BH || pos >= n_blocks) return;
  const int qb = qblock_order ? min(max(qblock_order[pos], 0), n_blocks - 1) : pos;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int qg = wave & 3;     // query group: rows 32*qg..+31 of the block
  const int kh = wave >> 2;    // key half: keys 64*kh..+63 of every tile
  const int n = lane & 31;     // query within the group (MFMA column)
  const int h = lane >> 5;     // lane half
  const int key0 = 64 * kh;

  const size_t head_off = (size_t)bh * L * kD * 2;    // bytes
  const __amdgpu_buffer_rsrc_t k_rsrc = head_rsrc(k + head_off, L * kD * 2);
  const __amdgpu_buffer_rsrc_t v_rsrc = head_rsrc(v + head_off, L * kD * 2);
  const int32_t* sel = block_idx + ((size_t)bh * n_blocks + qb) * topk;
  auto tile_block = [&](int t) { return min(max(sel[t], 0), n_blocks - 1); };

  // ---- Q^T operand: lane holds Q[query n][16*ks + 8*h + 0..7] for ks = 0..7
  // (rows past the end of a short last block load the last row and are not stored)
  const int qrow = qb * kBlock + qg * 32 + n;
  bf16x8 qf[8];
  {
    const unsigned char* qp = q + head_off + (size_t)min(qrow, L - 1) * kD * 2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + (16 * ks + 8 * h) * 2);
  }

  // ---- transpose-read addressing for V^T operands (per lane, loop invariant)
  // group g = lane/16 covers keys 4*(g/2)+0..3 (rows) x dims 16*(g%2)+0..15 of a 32-dim block.
  const int g = lane >> 4;
  const int rr = (lane & 15) >> 2, cc = lane & 3;
  const int tr_row0 = key0 + 4 * (g >> 1) + rr;                  // + 16*ks (+8)
  const int tr_col = 16 * (g & 1) + 4 * cc;                      // + 32*md   (elements)
  // Rows 16*ks + tr_row0 (+8) have the same swizzle for every ks (16*ks changes
  // neither row%4 nor (row/4)%4), so each (md, lo/hi) needs one base offset and
  // the k-step becomes an immediate offset of 16 rows * 256 bytes.
  int tr_off[2][4];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int md = 0; md < 4; ++md) {
      const int row = tr_row0 + 8 * hi;
      const int col = 32 * md + tr_col;
      tr_off[hi][md] = row * 256 + (((col >> 3) ^ swz(row)) << 4) + (col & 7) * 2;
    }

  f32x16 o[4];
#pragma unroll
  for (int md = 0; md < 4; ++md) o[md] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- prologue: K0, V0, K1 into LDS; S_0
  tile_dma(kbuf(0), k_rsrc, tile_block(0) * kTileBytes, wave, lane);
  tile_dma(vbuf(0), v_rsrc, tile_block(0) * kTileBytes, wave, lane);
  if (topk > 1) tile_dma(kbuf(1), k_rsrc, tile_block(1) * kTileBytes, wave, lane);
  __syncthreads();
  f32x16 sa[2], sb[2];
  compute_st(sa, kbuf(0), key0, qf, n, h);
  __syncthreads();   // every wave is done with K0 before iteration 0 refills its buffer

  auto step = [&](f32x16 (&scur)[2], f32x16 (&snext)[2], int t, int par) {
    const bool has_next = t + 1 < topk;
    // refill the buffers freed by the previous iteration: K_{t+2} and V_{t+1}
    if (t + 2 < topk) tile_dma(kbuf(par), k_rsrc, tile_block(t + 2) * kTileBytes, wave, lane);
    if (has_next) tile_dma(vbuf(par ^ 1), v_rsrc, tile_block(t + 1) * kTileBytes, wave, lane);
    // key half 0 computes the next S first, key half 1 after its softmax
    if (kh == 0 && has_next) compute_st(snext, kbuf(par ^ 1), key0, qf, n, h);

    // softmax on S_t (log2 domain)
    const int valid = L - tile_block(t) * kBlock;   // keys of the tile that exist (short last block)
    if (valid < kBlock) mask_missing_keys(scur, key0, h, valid);
    float mx = scur[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[mb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // a key half with no existing key yet keeps m = -inf, weights 0 and alpha 1
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    float lsum = 0.f;
    uint32_t pb[4][4];   // P^T operand per k-step (8 bf16 = 4 dwords)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(scur[mb][r], scale_log2, -m_sub));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(scur[mb][r + 1], scale_log2, -m_sub));
        lsum += p0 + p1;
        // register r of block mb holds key key0 + 32mb + 8(r/4) + 4h + r%4;
        // k-step ks = 2mb + r/8 takes r/4 even -> dwords 0,1 ; odd -> dwords 2,3
        const int ks = 2 * mb + (r >> 3);
        const int dw = ((r >> 2) & 1) * 2 + ((r & 3) >> 1);
        pb[ks][dw] = pack_bf16x2(p0, p1);
      }
    }
    l_run = l_run * alpha + lsum;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] *= alpha;
    }

    if (kh == 1 && has_next) compute_st(snext, kbuf(par ^ 1), key0, qf, n, h);

    // O^T += V^T P^T over this wave's 64 keys
    const unsigned char* vt = vbuf(par);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{pb[ks][0], pb[ks][1], pb[ks][2], pb[ks][3]});
      const unsigned char* vk = vt + ks * 16 * 256;
#pragma unroll
      for (int md = 0; md < 4; ++md) {
        const i16x4 lo = ds_read_tr(vk, tr_off[0][md]);
        const i16x4 hi = ds_read_tr(vk, tr_off[1][md]);
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
        o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[md], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
#pragma unroll
    for (int i = 0; i < 14; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 1);

    __syncthreads();   // also waits for this iteration's tile copies
  };

  // the last step is peeled: only it can meet the short last block (the largest index)
  int t = 0;
  for (; t + 1 < topk; t += 2) {
    step(sa, sb, t, 0);
    step(sb, sa, t + 1, 1);
  }
  if (t < topk) step(sa, sb, t, 0);

  // ---- merge the two key halves: half 1 publishes (m, l, O^T) through LDS (tile buffers are free)
  // one free 32 KiB tile buffer per query group holds its [66][64 lanes] floats (16.5 KiB)
  unsigned char* xbuf = qg == 0 ? k0s : (qg == 1 ? k1s : (qg == 2 ? v0s : v1s));
  float* mine = reinterpret_cast<float*>(xbuf);
  if (kh == 1) {
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[(md * 16 + r) * 64 + lane] = o[md][r];
    mine[64 * 64 + lane] = m_run;
    mine[65 * 64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 1) return;
  const float m1 = mine[64 * 64 + lane], l1 = mine[65 * 64 + lane];
  const float m = fmaxf(m_run, m1);
  const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
  const float l_lane = l_run * a0 + l1 * a1;
  const float l_tot = l_lane + __shfl_xor(l_lane, 32, 64);
  const float inv = 1.f / l_tot;
  const float c0 = a0 * inv, c1 = a1 * inv;
  if (qrow >= L) return;   // past the end of a short last block
  unsigned char* op = out + head_off + (size_t)qrow * kD * 2;
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // registers 4j..4j+3 hold dims 32md + 8j + 4h + 0..3 of query n
      const int dcol = 32 * md + 8 * j + 4 * h;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = o[md][4 * j + i] * c0 + mine[(md * 16 + 4 * j + i) * 64 + lane] * c1;
      u32x2 w{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      *reinterpret_cast<u32x2*>(op + dcol * 2) = w;
    }
  if (lse && h == 0) lse[(size_t)bh * L + qrow] = (m + __log2f(l_tot)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------------------
// Pair kernel: one workgroup = two query blocks A, B of one head (adjacent in the
// schedule, so their selections overlap), 8 waves: waves 0-3 serve A and 4-7 serve
// B (one of each per SIMD), each wave 32 queries.  The two ascending selections are
// held in registers and merged on the fly (one cursor for the copies, one for the
// compute); every K/V tile of the union is copied into LDS once and consumed by
// whichever block selected it.  Sparse gathers are bound by the bytes moved into
// the CUs (128 flop per tile byte for one 128-row query block); sharing tiles
// between two blocks whose selections overlap cuts those bytes by a third on the
// video workloads.
//
// Copies: a ring of five LDS slots of 32 KiB, each holding one half tile (64 keys
// of K and the same 64 keys of V).  A step consumes the two halves of one union
// tile while the next three half tiles are in flight, so a copy is issued one to
// two steps before it is needed.  The barrier opening a step waits only for this
// wave's copies of the step's own half tiles (s_waitcnt vmcnt leaves the younger
// copy in flight), not for every copy as a __syncthreads fence would.
//
// Compute per active wave and tile, ordered so that the matrix cores and the
// vector ALUs overlap inside the wave:
//   S0 = K0 Q^T, S1 = K1 Q^T      2 x 16 MFMA (64 keys each)
//   softmax(S0)                   VALU, runs under the S1 products
//   O^T += V0^T P0^T              16 MFMA, runs under softmax(S1)
//   O^T += V1^T P1^T              16 MFMA
// The running max is raised per half (lazily, see above), so O is rescaled
// before each half's product only when a raise occurred.
constexpr int kSlots = 5;
constexpr int kHalfBytes = 64 * kD * 2;        // 64 rows of K (or V): 16 KiB
constexpr int kSlotBytes = 2 * kHalfBytes;     // K half, then V half
constexpr int kCopiesPerHalf = 4;              // global_load_lds per wave per half tile
constexpr int kNoBlock = 0x7fffffff;
constexpr int kListRegs = 2;                   // selections of up to 128 blocks in registers

// s_waitcnt immediate (gfx9 layout): vmcnt <= n, lgkmcnt == 0, expcnt unconstrained.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Empty asm that takes x in a register at this point of the program: keeps a value's
// computation in the scheduling slot where it is written (the slots are separated by
// scheduling fences), instead of letting it drift towards its first use.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }


// Copy 64 rows of K and the same 64 rows of V into one slot (wave w: segments w, w+8),
// starting at byte `off` of the head.  MUBUF direct-to-LDS loads: unlike the FLAT
// form, they leave the compiler free to wait for LDS reads individually.
__device__ __forceinline__ void half_dma(unsigned char* lds, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                         int off, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int seg = wave + 8 * i;
    const int row = 4 * seg + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);
    const int voff = off + row * 256 + c * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void*)(lds + seg * 1024), 16,
                                             voff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(lds + kHalfBytes + seg * 1024),
                                             16, voff, 0, 0, 0);
  }
}

// Wait until this wave's copies of the step's half tiles have landed (the one
// younger half tile stays in flight) and its LDS reads are done, then barrier.  The
// empty asm statements keep the compiler from moving memory accesses across the
// barrier.
__device__ __forceinline__ void wait_copies_and_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerHalf));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_pair_kernel(
    const unsigned char* __restrict__ q, const unsigned char* __restrict__ k,
    const unsigned char* __restrict__ v, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ qblock_order, int BH, int L, int n_blocks, int topk, int n_pairs,
    int per_xcd, float scale_log2, unsigned char* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) unsigned char sl0[kSlotBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sl1[kSlotBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sl2[kSlotBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sl3[kSlotBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sl4[kSlotBytes];
  auto slot = [&](int s) { return s == 0 ? sl0 : s == 1 ? sl1 : s == 2 ? sl2 : s == 3 ? sl3 : sl4; };

  // ---- work mapping (XCD-aware, head-major across the whole chip)
  const int wg = blockIdx.x;
  const int xcd = wg % kXcds;
  const int wslot = wg / kXcds;
  const int bh = wslot / per_xcd;
  const int pr = xcd * per_xcd + wslot % per_xcd;
  if (bh >= BH || pr >= n_pairs) return;
  auto qblock_at = [&](int pos) {
    return qblock_order ? min(max(qblock_order[pos], 0), n_blocks - 1) : pos;
  };
  const int qa = qblock_at(2 * pr);
  const int qbb = 2 * pr + 1 < n_blocks ? qblock_at(2 * pr + 1) : -1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int grp = wave >> 2;   // 0: block A, 1: block B
  const int qg = wave & 3;     // rows 32*qg..+31 of the wave's block
  const int n = lane & 31;
  const int h = lane >> 5;
  const int myq = grp ? qbb : qa;

  const size_t head_off = (size_t)bh * L * kD * 2;
  const __amdgpu_buffer_rsrc_t k_rsrc = head_rsrc(k + head_off, L * kD * 2);
  const __amdgpu_buffer_rsrc_t v_rsrc = head_rsrc(v + head_off, L * kD * 2);

  // ---- Q^T operand of the wave's 32 queries (loaded before any tile copy; rows past
  // the end of a short last block load the last row and are not stored)
  const int qrow = (myq >= 0 ? myq : 0) * kBlock + qg * 32 + n;
  bf16x8 qf[8];
  {
    const unsigned char* qp = q + head_off + (size_t)min(qrow, L - 1) * kD * 2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + (16 * ks + 8 * h) * 2);
  }

  // ---- the two ascending selections, held in registers: lane l keeps entries
  // l and 64+l (kNoBlock past the end); read back with v_readlane
  const int32_t* sa = block_idx + ((size_t)bh * n_blocks + qa) * topk;
  const int32_t* sb = block_idx + ((size_t)bh * n_blocks + (qbb >= 0 ? qbb : qa)) * topk;
  const int nsel_b = qbb >= 0 ? topk : 0;
  int la[kListRegs], lb[kListRegs];
#pragma unroll
  for (int r = 0; r < kListRegs; ++r) {
    const int i = 64 * r + lane;
    la[r] = i < topk ? min(max(sa[i], 0), n_blocks - 1) : kNoBlock;
    lb[r] = i < nsel_b ? min(max(sb[i], 0), n_blocks - 1) : kNoBlock;
  }
  auto entry = [&](const int (&lst)[kListRegs], int i) {   // i wave-uniform
    const int ln = i & 63, r = i >> 6;
    int x = kNoBlock;
#pragma unroll
    for (int t = 0; t < kListRegs; ++t) {
      const int y = __builtin_amdgcn_readlane(lst[t], ln);
      x = r == t ? y : x;
    }
    return x;
  };
  auto head = [&](const int (&lst)[kListRegs], int i, int cnt) { return i < cnt ? entry(lst, i) : kNoBlock; };
  // A short last block (L not a multiple of 128) is the last entry of any selection
  // that contains it; it is left out of the main walk and handled after it with its
  // missing keys masked, so the main loop carries no masking code.
  const int last = n_blocks - 1;
  const bool short_last = L % kBlock != 0;
  const bool short_a = short_last && entry(la, topk - 1) == last;
  const bool short_b = short_last && nsel_b > 0 && entry(lb, nsel_b - 1) == last;
  const int cnt_a = topk - (short_a ? 1 : 0), cnt_b = nsel_b - (short_b ? 1 : 0);
  struct Cursor { int ia, ib, ja, jb; };
  // merge step: the smaller head (both when equal) is the next tile of the union
  auto advance = [&](Cursor& c, int& j, bool& fa, bool& fb) {
    j = min(c.ja, c.jb);
    if (j == kNoBlock) return false;
    fa = c.ja == j;
    fb = c.jb == j;
    if (fa) c.ja = head(la, ++c.ia, cnt_a);
    if (fb) c.jb = head(lb, ++c.ib, cnt_b);
    return true;
  };
  Cursor c_copy{0, 0, head(la, 0, cnt_a), head(lb, 0, cnt_b)};
  Cursor c_comp = c_copy;

  // ---- copy side: half tile w = 2 * (union position) + (key half)
  int j_copy = 0;
  bool copy_done = false;
  // Every step issues exactly two half-tile copies: past the end of the union the
  // last tile is copied again into the free slot (never read).  A fixed count keeps
  // the compiler's model of the copies in flight exact, so it adds no wait of its own
  // before the LDS reads.
  auto issue = [&](int w, unsigned char* buf) __attribute__((always_inline)) {
    if (!copy_done && (w & 1) == 0) {
      int j;
      bool fa, fb;
      if (advance(c_copy, j, fa, fb)) j_copy = j; else copy_done = true;
    }
    half_dma(buf, k_rsrc, v_rsrc, j_copy * kTileBytes + (w & 1) * kHalfBytes, wave, lane);
  };

  // ---- transpose-read offsets for V^T operands (see the single-block kernel)
  const int g = lane >> 4;
  const int rr = (lane & 15) >> 2, cc = lane & 3;
  const int tr_row0 = 4 * (g >> 1) + rr;
  const int tr_col = 16 * (g & 1) + 4 * cc;
  int tr_off[2][4];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int md = 0; md < 4; ++md) {
      const int row = tr_row0 + 8 * hi;
      const int col = 32 * md + tr_col;
      tr_off[hi][md] = row * 256 + (((col >> 3) ^ swz(row)) << 4) + (col & 7) * 2;
    }

  f32x16 o[4];
#pragma unroll
  for (int md = 0; md < 4; ++md) o[md] = f32x16{};
  float m_use = -INFINITY, l_run = 0.f;

  // ---- per active tile: products and softmax interleaved inside the wave.  Each
  // slot below is one matrix-core product plus the operand reads for a later
  // product plus a share of the vector work of the previous half's softmax; a
  // scheduling fence between slots keeps that interleave (the matrix core runs a
  // product while the vector ALU works on independent data).
  const uint32_t ones_bf16x2 = 0x3f803f80u;
  // K operand of score product i (0..31): half i/16, k-step (i%16)/2, key block i%2
  auto kread = [&](const unsigned char* k0, const unsigned char* k1, int i) {
    const unsigned char* kt = i < 16 ? k0 : k1;
    return *reinterpret_cast<const bf16x8*>(kt + lds_off(32 * (i & 1) + n, 2 * ((i & 15) >> 1) + h));
  };
  // V^T operand of value product i (0..15 of one half): k-step i/4, dim block i%4
  auto vread = [&](const unsigned char* vt, int i) {
    const unsigned char* vk = vt + (i >> 2) * 16 * 256;
    const u32x2 lo = __builtin_bit_cast(u32x2, ds_read_tr(vk, tr_off[0][i & 3]));
    const u32x2 hi = __builtin_bit_cast(u32x2, ds_read_tr(vk, tr_off[1][i & 3]));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  // softmax of one half (32 scores per lane), in 16 pieces: 0-1 row max, 3 new
  // reference max (raised lazily, see above), 4-15 probabilities (bf16 pairs),
  // their sum (dot with ones, i.e. the sum of the rounded weights the products use)
  struct Soft { float mx, other, alpha, lsum; bool up; };
  auto soft_piece = [&](int j, const f32x16 (&s)[2], uint32_t (&pb)[4][4], Soft& st) {
    if (j == 0) {
      st.mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) st.mx = fmaxf(st.mx, s[0][r]);
      pin(st.mx);
    } else if (j == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st.mx = fmaxf(st.mx, s[1][r]);
      st.other = __shfl_xor(st.mx, 32, 64);
      pin(st.mx);
    } else if (j == 3) {
      const float mx = fmaxf(st.mx, st.other) * scale_log2;
      st.up = mx > m_use + kRescaleSlack;
      const float m_new = st.up ? mx : m_use;
      st.alpha = st.up ? __builtin_amdgcn_exp2f(m_use - m_new) : 1.f;
      m_use = m_new;
      st.lsum = 0.f;
      pin(m_use);
      pin(st.alpha);
    } else if (j >= 4) {
      const int x = j - 4;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int pp = t == 0 ? x : 12 + x;   // register pair: pieces 4-7 take two
        if (t == 1 && x >= 4) break;
        const int mb = pp >> 3, r = 2 * (pp & 7);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[mb][r], scale_log2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[mb][r + 1], scale_log2, -m_use));
        uint32_t w = pack_bf16x2(p0, p1);
        pin(w);
        pb[2 * mb + (r >> 3)][((r >> 2) & 1) * 2 + ((r & 3) >> 1)] = w;
        st.lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                                  __builtin_bit_cast(bf16x2, ones_bf16x2), st.lsum, false);
      }
    }
  };
  auto soft_finish = [&](Soft& st) {
    pin(st.lsum);
    l_run = l_run * st.alpha + st.lsum;
    if (__ballot(st.up)) {
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] *= st.alpha;
    }
  };
  // MASK (compile-time): the tile is a short last block with `valid` keys
  auto consume = [&](auto mask_tag, const unsigned char* h0, const unsigned char* h1, int valid)
                     __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 s0[2], s1[2];
    uint32_t pb0[4][4], pb1[4][4];
    Soft st0, st1;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s0[mb] = f32x16{};
      s1[mb] = f32x16{};
    }
    // S0 = K0 Q^T and S1 = K1 Q^T (operand reads four products ahead); softmax(S0)
    // runs in the slots of S1
    bf16x8 ka[5];
#pragma unroll
    for (int i = 0; i < 4; ++i) ka[i] = kread(h0, h1, i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + 4 < 32) ka[(i + 4) % 5] = kread(h0, h1, i + 4);
      const int ks = (i & 15) >> 1, mb = i & 1;
      if (i < 16) {
        s0[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % 5], qf[ks], s0[mb], 0, 0, 0);
      } else {
        if (MASK && i == 16) mask_missing_keys(s0, 0, h, valid);
        s1[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % 5], qf[ks], s1[mb], 0, 0, 0);
        soft_piece(i - 16, s0, pb0, st0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    soft_finish(st0);
    // O^T += V0^T P0^T (operand reads two products ahead); softmax(S1) in its slots
    const unsigned char* v0 = h0 + kHalfBytes;
    const unsigned char* v1 = h1 + kHalfBytes;
    if (MASK) mask_missing_keys(s1, 64, h, valid);
    bf16x8 va[3];
    va[0] = vread(v0, 0);
    va[1] = vread(v0, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) va[(i + 2) % 3] = vread(v0, i + 2);
      const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{pb0[i >> 2][0], pb0[i >> 2][1], pb0[i >> 2][2], pb0[i >> 2][3]});
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 3], b, o[i & 3], 0, 0, 0);
      soft_piece(i, s1, pb1, st1);
      __builtin_amdgcn_sched_barrier(0);
    }
    soft_finish(st1);
    // O^T += V1^T P1^T
    va[0] = vread(v1, 0);
    va[1] = vread(v1, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) va[(i + 2) % 3] = vread(v1, i + 2);
      const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{pb1[i >> 2][0], pb1[i >> 2][1], pb1[i >> 2][2], pb1[i >> 2][3]});
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 3], b, o[i & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // step u consumes half tiles 2u, 2u+1 (slots (2u)%5, (2u+1)%5) and refills the
  // two slots released by step u-1 with half tiles 2u+3, 2u+4
  bool use_a = false, use_b = false;
  auto step = [&](int u, int s0, int s1, int r0, int r1) __attribute__((always_inline)) {
    int j;
    if (!advance(c_comp, j, use_a, use_b)) return false;
    wait_copies_and_barrier();
    issue(2 * u + 3, slot(r0));
    issue(2 * u + 4, slot(r1));
    if (myq >= 0 && (grp ? use_b : use_a)) consume(std::false_type{}, slot(s0), slot(s1), kBlock);
    return true;
  };

  issue(0, sl0);
  issue(1, sl1);
  issue(2, sl2);
  for (int u = 0;; u += kSlots) {
    if (!step(u, 0, 1, 3, 4)) break;
    if (!step(u + 1, 2, 3, 0, 1)) break;
    if (!step(u + 2, 4, 0, 2, 3)) break;
    if (!step(u + 3, 1, 2, 4, 0)) break;
    if (!step(u + 4, 3, 4, 1, 2)) break;
  }

  // ---- the short last block, if selected: copied once all other copies have landed
  if (short_a || short_b) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __syncthreads();
    half_dma(sl0, k_rsrc, v_rsrc, last * kTileBytes, wave, lane);
    half_dma(sl1, k_rsrc, v_rsrc, last * kTileBytes + kHalfBytes, wave, lane);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __syncthreads();
    if (myq >= 0 && (grp ? short_b : short_a)) consume(std::true_type{}, sl0, sl1, L - last * kBlock);
  }

  // ---- epilogue: O = O^T / l
  if (myq < 0 || qrow >= L) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  unsigned char* op = out + head_off + (size_t)qrow * kD * 2;
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dcol = 32 * md + 8 * j + 4 * h;
      u32x2 w{pack_bf16x2(o[md][4 * j] * inv, o[md][4 * j + 1] * inv),
              pack_bf16x2(o[md][4 * j + 2] * inv, o[md][4 * j + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + dcol * 2) = w;
    }
  if (lse && h == 0) lse[(size_t)bh * L + qrow] = (m_use + __log2f(l_tot)) * 0.69314718055994530942f;
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, int BH, int L, int topk,
                           const int32_t* block_idx, const int32_t* qblock_order, float scale, void* out,
                           float* lse, hipStream_t stream) {
  (void)hipGetLastError();   // report this launch only, not an earlier unrelated error
  const int n_blocks = (L + kBlock - 1) / kBlock;   // the last block may be short
  const float scale_log2 = scale * 1.4426950408889634f;
  if (topk <= 64 * kListRegs) {
    const int n_pairs = (n_blocks + 1) / 2;
    const int per_xcd = (n_pairs + kXcds - 1) / kXcds;
    const long long grid = (long long)kXcds * per_xcd * BH;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fwd_bf16_pair_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       static_cast<const unsigned char*>(q), static_cast<const unsigned char*>(k),
                       static_cast<const unsigned char*>(v), block_idx, qblock_order, BH, L, n_blocks, topk,
                       n_pairs, per_xcd, scale_log2, static_cast<unsigned char*>(out), lse);
    return hipGetLastError();
  }
  const int per_xcd = (n_blocks + kXcds - 1) / kXcds;
  const long long grid = (long long)kXcds * per_xcd * BH;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const unsigned char*>(q), static_cast<const unsigned char*>(k),
                     static_cast<const unsigned char*>(v), block_idx, qblock_order, BH, L, n_blocks, topk, per_xcd,
                     scale_log2, static_cast<unsigned char*>(out), lse);
  return hipGetLastError();
}

}  // namespace sol_attn
