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
//                      of one lane pair (l, l^32).
//   softmax            in the log2 domain against the running max m of the wave's
//                      key half: p = 2^(s*scale*log2(e) - m) (v_exp_f32), l += sum p.
//                      The max is not recomputed per tile: the common factor 2^-m
//                      cancels in O/l, so only a weight sum above 2^15 (a score that
//                      rose far above m, or the first tile) makes the wave find the
//                      row max, raise m and rescale O and l.
//   O^T += V_j^T P^T   16 MFMA 32x32x16: the S^T accumulator layout already is
//                      the B-operand layout of P^T (after bf16 rounding) for a
//                      fixed permutation of the 16 keys of each k-step; the A
//                      operand V^T is read with ds_read_b64_tr_b16, whose
//                      16-lane transpose delivers 4 consecutive keys of one
//                      column per lane, in the same key permutation.
//
// Two waves share each SIMD: the two key halves of the same 32 queries.  Each step
// (one tile) has two halves; in each, one wave of the pair runs its matrix phase --
// S_{t+1} and O += V_t^T P_t^T, 32 products, at raised issue priority -- while the
// other runs its softmax (the P it accumulates next); the roles swap in the second
// half.  Key half 0 takes the matrix phase first, key half 1 second; the loop is
// compiled once per key half so each wave runs straight-line code for its role.
// Without this the older wave wins issue arbitration, runs ahead, and every step
// ends with one wave alone on the SIMD (measured: the younger waves' steps set the
// pace while the older ones idled a third of the time at the barrier).
//
// Copies: LDS holds three K tiles and two V tiles (5 x 32 KiB, the whole 160 KiB):
// K_j in K buffer j%3 (read for S_j in step j-1), V_j in V buffer j%2 (read in step
// j).  Step t refills V(t-1)'s buffer with V(t+1) and K(t)'s with K(t+3); each wave
// issues its share of both from its softmax phase (V before the weights, K after),
// so the matrix-phase wave only reads LDS.  The wait opening a step (vmcnt <= 4)
// leaves only this wave's K(t+3) copies in flight, and the barrier after it makes
// every wave's copies visible and frees the two buffers.  A step's block indices are
// scalar loads issued before that wait, which drains the scalar/LDS counter anyway:
// loaded later, their wait would also drain the operand reads running ahead of the
// products.  Past the end of the list the last tile is copied again into the free
// buffer (never read), keeping the copies per step fixed; each tile gets its own
// buffer resource, whose range makes rows past the end of a short last block read as
// zero.  The iterations are unrolled six at a time (periods 3 and 2), so every
// buffer is a compile-time choice and the compiler adds no waits of its own.
//
// Where the time goes (1344x768 workload, per step and CU): 128 KiB of K operand
// reads, 128 KiB of transposed V reads and 64 KiB of copies written land on an LDS
// that moves 128 B per clock for 16-byte reads and 78-120 B per clock for transposed
// reads: at least ~2500 clocks (~2630 at the transposed rate of 8 waves), against 2048
// clocks of matrix-core work; a step measures ~2650 clocks.
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
//
// Cube blocks (3-D boxes of the latent grid, 128 tokens each) are read in place from
// the frame-major tensors: a tile's 16-byte copies are addressed from the box's first
// token plus each copy row's offset inside the box (by rows of bx consecutive tokens),
// which leaves the LDS tile exactly as for 128 consecutive tokens; Q rows, O rows and
// lse entries likewise sit at their frame-major positions.  No reordered copy of Q, K,
// V or O is made.
#include <type_traits>

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
// s_waitcnt immediate (gfx9 layout): vmcnt <= n, lgkmcnt == 0, expcnt unconstrained.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
// how many products ahead of the matrix core the K and transposed V operand reads run
// (deeper is slower: the reads then queue on the LDS, which is the busier unit)
constexpr int kKAhead = 4;
constexpr int kVAhead = 3;

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
//
// Each tile gets its own buffer resource whose base is the tile's first token and whose
// range is the bytes the tile may read: rows past the end of the head (the missing rows
// of a short last block) are outside it and read as zero.  The per-lane byte offsets
// inside the tile are loop invariants, so a copy costs no vector arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const unsigned char* head, int off, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(head) + off, (short)0, bytes, 0x00020000);
}

// First token of key/query block j, and offset from it of the block's row r: blocks of
// 128 consecutive tokens, or boxes of the latent grid read in place (cube blocks).
template <bool kCube>
__device__ __forceinline__ int block_first_token(const BoxGeom& g, int j) {
  return kCube ? g.first_token(j) : j * kBlock;
}
template <bool kCube>
__device__ __forceinline__ int row_token_offset(const BoxGeom& g, int r) {
  return kCube ? g.row_offset(r) : r;
}

// Copy segment i (of wave, wave+8, wave+16, wave+24) of a tile; laneoff[i] = byte offset,
// from the tile's first token, of the 16 bytes this lane fetches for that segment.
__device__ __forceinline__ void tile_dma_seg(unsigned char* lds, __amdgpu_buffer_rsrc_t r, const int (&laneoff)[4],
                                             int wave, int i) {
  const int seg = wave + 8 * i;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds + seg * 1024), 16,
                                           laneoff[i], 0, 0, 0);
}

__device__ __forceinline__ void tile_dma(unsigned char* lds, __amdgpu_buffer_rsrc_t r, const int (&laneoff)[4],
                                         int wave) {
#pragma unroll
  for (int i = 0; i < 4; ++i) tile_dma_seg(lds, r, laneoff, wave, i);
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

// Weights p = 2^(s*scale_log2 - m) of this lane's 32 scores, rounded to bf16 into the P^T
// operand layout (pb[k-step][dword]); returns this lane's float32 sum of the weights.
// Score register r of s[mb] is key 32mb + 8(r/4) + 4h + r%4: k-step 2mb + r/8 takes
// registers 8(r/8)..+7, dword 2((r/4)%2) + (r%4)/2 of it holds the pair (r, r+1).
__device__ __forceinline__ float softmax_weights(const f32x16 (&s)[2], float scale_log2, float m,
                                                 uint32_t (&pb)[4][4]) {
  float acc0 = 0.f, acc1 = 0.f;   // two chains of additions
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[mb][r], scale_log2, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[mb][r + 1], scale_log2, -m));
      pb[2 * mb + (r >> 3)][((r >> 2) & 1) * 2 + ((r & 3) >> 1)] = pack_bf16x2(p0, p1);
      if (r & 2) acc1 += p0 + p1; else acc0 += p0 + p1;
    }
  // the packed weights are formed here, not next to the products that read them: 16
  // registers instead of 32 live until then, and no conversions in the matrix phase
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) asm volatile("" : "+v"(pb[ks][dw]));
  return acc0 + acc1;
}

// S^T (64 keys of this wave's half x 32 queries) = K_half . Q^T.
__device__ __forceinline__ void compute_st(f32x16 (&s)[2], const unsigned char* kt, int key0,
                                           const bf16x8 (&qf)[8], int n, int h) {
  // the two 32-key accumulators alternate, so consecutive products are independent
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int row = key0 + 32 * mb + n;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + lds_off(row, 2 * ks + h));
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0, 0);
    }
  }
  // operand reads run kKAhead products ahead of the matrix core (deeper costs registers)
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kKAhead, 0);
#pragma unroll
  for (int i = 0; i < 16 - kKAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, kKAhead, 0);
}

template <bool kCube>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const unsigned char* __restrict__ q, const unsigned char* __restrict__ k,
    const unsigned char* __restrict__ v, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ qblock_order, int BH, int L,
    int n_blocks, int topk, int per_xcd, float scale_log2, unsigned char* __restrict__ out,
    float* __restrict__ lse, BoxGeom geom) {
  // Four separate LDS arrays (not one): the compiler can then prove that reads of
  // one buffer never alias the in-flight direct-to-LDS copies into another, and
  // does not insert a wait for those copies in the middle of the iteration.
  __shared__ __attribute__((aligned(16))) unsigned char k0s[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char k1s[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char k2s[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v0s[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v1s[kTileBytes];
  auto kbuf = [&](int p) { return p == 0 ? k0s : p == 1 ? k1s : k2s; };
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
  const unsigned char* k_head = k + head_off;
  const unsigned char* v_head = v + head_off;
  const int32_t* sel = block_idx + ((size_t)bh * n_blocks + qb) * topk;
  auto tile_block = [&](int t) { return min(max(sel[t], 0), n_blocks - 1); };

  // ---- Q^T operand: lane holds Q[query n][16*ks + 8*h + 0..7] for ks = 0..7
  // (rows past the end of a short last block load the last row and are not stored)
  const int qrow = block_first_token<kCube>(geom, qb) + row_token_offset<kCube>(geom, qg * 32 + n);
  // byte offset, from a tile's first token, of the 16 bytes this lane copies in each of
  // its copy segments (its row, and the logical chunk the swizzle puts at lane%16)
  int laneoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * (wave + 8 * i) + (lane >> 4);
    laneoff[i] = row_token_offset<kCube>(geom, row) * kD * 2 + (((lane & 15) ^ swz(row)) << 4);
  }
  auto tile_off = [&](int j) { return block_first_token<kCube>(geom, j) * kD * 2; };
  // bytes a tile starting at byte `off` may read: 128 rows (fewer for a short last block);
  // a box's rows are spread over the head, which it never passes
  const int head_bytes = L * kD * 2;
  auto tile_bytes = [&](int off) { return kCube ? head_bytes - off : min(head_bytes - off, kTileBytes); };
  auto k_tile = [&](int off) { return tile_rsrc(k_head, off, tile_bytes(off)); };
  auto v_tile = [&](int off) { return tile_rsrc(v_head, off, tile_bytes(off)); };
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
  f32x16 st[2];         // S^T of the tile this wave scores next
  uint32_t pb[4][4];    // P^T operand (8 bf16 = 4 dwords per k-step) of the tile it accumulates next

  // Softmax of the scores in st for key block `tb` (log2 domain): p = 2^(s*scale_log2 - m_run)
  // against the running max, rounded to bf16 into pb.  The max is not recomputed per tile:
  // any m works (the common factor 2^-m cancels between O and l) as long as no weight
  // overflows.  So the weights are formed with the current m_run, and only if some lane's
  // sum of its 32 weights exceeds 2^15 (or is not finite: the first tile, where m_run =
  // -inf) does the wave take the exact path -- row max, m_run raised to it, O and l
  // rescaled, weights formed again (then <= 1).  Every weight stays <= 2^15.
  auto softmax_tile = [&](int tb) __attribute__((always_inline)) {
    const int valid = kCube ? kBlock : L - tb * kBlock;   // keys that exist (short last block)
    if (valid < kBlock) mask_missing_keys(st, key0, h, valid);
    float lsum = softmax_weights(st, scale_log2, m_run, pb);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(lsum <= 32768.f)) != 0, 0)) {
      float mx = st[0][0];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[mb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // a key half with no existing key yet keeps m = -inf, weights 0 and alpha 1
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] *= alpha;
      lsum = softmax_weights(st, scale_log2, m_new == -INFINITY ? 0.f : m_new, pb);
    }
    l_run += lsum;
  };

  // ---- prologue: K0, K1, K2 and V0 into LDS; S_0 (and, for key half 0, P_0)
  // K(j) lives in K buffer j%3 and is read in step j-1 (for S_j), V(j) in V buffer j%2,
  // read in step j.  Step t refills the V buffer of V(t-1) with V(t+1) and the K buffer of
  // K(t) (read in step t-1) with K(t+3), one quarter per k-step of the P.V products; V's
  // copies are issued first, so the wait opening step t+1 (vmcnt <= 4) leaves only this
  // wave's four K(t+3) copies in flight.  Past the end of the list the last tile is
  // copied again into the free buffer (never read), keeping the copies per step fixed.
  auto blk = [&](int t) { return tile_block(min(t, topk - 1)); };
  tile_dma(kbuf(0), k_tile(tile_off(blk(0))), laneoff, wave);
  tile_dma(vbuf(0), v_tile(tile_off(blk(0))), laneoff, wave);
  tile_dma(kbuf(1), k_tile(tile_off(blk(1))), laneoff, wave);
  tile_dma(kbuf(2), k_tile(tile_off(blk(2))), laneoff, wave);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8));      // K0 and V0 landed (K1, K2 may fly)
  __syncthreads();
  compute_st(st, kbuf(0), key0, qf, n, h);
  int cur_blk = blk(0);   // block of tile t, read (scalar) by the step before: no vector load in the loop


  // Step t in two halves separated by a barrier.  In each half one wave of a SIMD's pair
  // runs its matrix phase -- S_{t+1} = K(t+1) Q^T and O^T += V(t)^T P_t^T, 32 products --
  // at raised issue priority, while the other runs its vector phase (the softmax of the
  // tile it accumulates next); the roles swap in the second half.  Key half 0 takes the
  // matrix phase first (its P_t was formed in the previous step's second half), key half
  // 1 second (its P_t is formed in the first half).  The barrier keeps the pair in
  // opposite phases: without it the older wave wins issue arbitration, runs ahead, and
  // the pair ends each step with one wave alone on the SIMD.  The loop is compiled once
  // per key half (KH), so each wave runs straight-line code for its own role.
  auto run = [&](auto khc) __attribute__((always_inline)) {
    constexpr int KH = decltype(khc)::value;
    if (KH == 0) softmax_tile(cur_blk);

    auto matrix_phase = [&](bool has_next, unsigned char* k_next, unsigned char* v_cur)
                            __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(1);
      if (has_next) compute_st(st, k_next, key0, qf, n, h);
      __builtin_amdgcn_sched_barrier(0);
      // O^T += V^T P^T over this wave's 64 keys
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{pb[ks][0], pb[ks][1], pb[ks][2], pb[ks][3]});
        const unsigned char* vk = v_cur + ks * 16 * 256;
#pragma unroll
        for (int md = 0; md < 4; ++md) {
          const i16x4 lo = ds_read_tr(vk, tr_off[0][md]);
          const i16x4 hi = ds_read_tr(vk, tr_off[1][md]);
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
          o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[md], 0, 0, 0);
        }
      }
      // transposed V reads run kVAhead products ahead (two reads per product)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kVAhead, 1);
#pragma unroll
      for (int i = 0; i < 16 - kVAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kVAhead, 1);
      __builtin_amdgcn_s_setprio(0);
    };

    auto step = [&](int t, unsigned char* k_next, unsigned char* k_free, unsigned char* v_cur,
                    unsigned char* v_free) __attribute__((always_inline)) {
      const bool has_next = t + 1 < topk;
      const int blk_t = cur_blk;
      // The step's block indices are scalar loads issued before the wait below, which
      // already drains the scalar/LDS counter: loaded later, their own wait would also
      // drain the operand reads running ahead of the products.
      const int blk_t1 = blk(t + 1);
      const int blk_t3 = blk(t + 3);
      cur_blk = blk_t1;
      // this wave's copies of K(t+1) and V(t) have landed (only its four copies of
      // K(t+2), the youngest, may still be in flight) and its LDS reads are done; after
      // the barrier every wave's copies are in LDS and every wave is done with K(t)
      // (read for S_t in step t-1) and V(t-1), whose buffers this step refills
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(4));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int k3_off = tile_off(blk_t3), v_off = tile_off(blk_t1);
      auto mid_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      };
      if (KH == 0) {
        matrix_phase(has_next, k_next, v_cur);
        mid_barrier();
        tile_dma(v_free, v_tile(v_off), laneoff, wave);
        if (has_next) softmax_tile(blk_t1);          // P_{t+1}
        tile_dma(k_free, k_tile(k3_off), laneoff, wave);
      } else {
        tile_dma(v_free, v_tile(v_off), laneoff, wave);
        softmax_tile(blk_t);                          // P_t
        tile_dma(k_free, k_tile(k3_off), laneoff, wave);
        mid_barrier();
        matrix_phase(has_next, k_next, v_cur);
      }
    };

    // six steps per round: K buffers cycle with period 3, V buffers with 2
    for (int t = 0; t < topk; t += 6) {
      step(t, k1s, k0s, v0s, v1s);
      if (t + 1 >= topk) break;
      step(t + 1, k2s, k1s, v1s, v0s);
      if (t + 2 >= topk) break;
      step(t + 2, k0s, k2s, v0s, v1s);
      if (t + 3 >= topk) break;
      step(t + 3, k1s, k0s, v1s, v0s);
      if (t + 4 >= topk) break;
      step(t + 4, k2s, k1s, v0s, v1s);
      if (t + 5 >= topk) break;
      step(t + 5, k0s, k2s, v1s, v0s);
    }
  };
  if (kh == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
  // every copy landed and every wave done with the tile buffers before they are reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __syncthreads();

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

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, int BH, int L, int topk,
                           const int32_t* block_idx, const int32_t* qblock_order, const BoxGeom* cube,
                           float scale, void* out, float* lse, hipStream_t stream) {
  (void)hipGetLastError();   // report this launch only, not an earlier unrelated error
  const int n_blocks = (L + kBlock - 1) / kBlock;   // the last block may be short
  const float scale_log2 = scale * 1.4426950408889634f;
  const int per_xcd = (n_blocks + kXcds - 1) / kXcds;
  const long long grid = (long long)kXcds * per_xcd * BH;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const BoxGeom geom = cube ? *cube : BoxGeom{};
  const auto* qs = static_cast<const unsigned char*>(q);
  const auto* ks = static_cast<const unsigned char*>(k);
  const auto* vs = static_cast<const unsigned char*>(v);
  auto* os = static_cast<unsigned char*>(out);
  if (cube)
    hipLaunchKernelGGL(fwd_bf16_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, qs, ks, vs,
                       block_idx, qblock_order, BH, L, n_blocks, topk, per_xcd, scale_log2, os, lse, geom);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, qs, ks, vs,
                       block_idx, qblock_order, BH, L, n_blocks, topk, per_xcd, scale_log2, os, lse, geom);
  return hipGetLastError();
}

}  // namespace sol_attn
