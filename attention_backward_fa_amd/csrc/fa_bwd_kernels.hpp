// fa_bwd_kernels.hpp -- device code of the attention backward on gfx950.
//   fa_bwd_pre     per (token, head) row: D = rowsum(O*dO) (step 4 of the
//                  PyPTO-Gym SK-16 article's per-tile math, section 3.1),
//                  the base-2 log-sum-exp of the forward's (m, l), a zeroed
//                  fp32 dQ accumulator row (single-pass form), and zeroed
//                  dQ/dK/dV rows outside every sequence. HBM bound.
//   fa_bwd_main    single-pass form, one workgroup per (kv tile, head,
//                  sequence): keeps the tile's K, V and its fp32 dK, dV
//                  accumulators in registers, streams the q tiles through LDS
//                  and runs the five GEMMs of steps 1, 3, 6, 7, 8 on bf16 MFMA
//                  with the softmax recompute and dS (steps 2, 5) on the VALU;
//                  dQ partial sums go to the fp32 accumulator with global
//                  atomics, or (split-and-reduce form) into the buffer of
//                  one of 8 kv-tile splits with plain loads and stores.
//   fa_bwd_dq_cast single-pass form: dQ = bf16(scale * accumulator). HBM bound.
//   fa_bwd_split_reduce  split-and-reduce form: sums the 8 split buffers in a
//                  fixed order and casts dQ to bf16. HBM bound.
//   fa_bwd_dkdv    recompute form, kv-outer: steps 1-3 and 5-7 with two
//                  waves per SIMD, each holding its keys' K rows in registers,
//                  in eight-wave or four-wave workgroups; dK, dV written once
//                  per kv tile.
//   fa_bwd_dq      recompute form, q-outer: recomputes S^T and dP^T and
//                  accumulates dQ (step 8) in registers; no atomics.
//   fa_fwd_fill,   the forward that produces O, m, l (the statistics step 2
//   fa_fwd         reads), for callers without one of their own.
// The recompute kernels and the forward also take grouped K/V heads, a
// sliding window (each query sees keys (i - w, i]) and any head dims that are
// multiples of 8 up to 256, separately for Q/K and for V/O/dO (latent
// attention): they are compiled for padded dims DQ, DV in {64, 128, 192, 256}, and
// the columns from a head dim up to its padded dim are loaded as zeros and
// never stored.
#pragma once
#include <type_traits>

#include "cdna4.hpp"

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;

// First row and valid length of sequence b (layout in include/fa_bwd.h).
__device__ __forceinline__ void seq_of(const int* cu, int b, int padded, int max_seqlen, int64_t& start,
                                       int& len) {
  const int c0 = cu[b], c1 = cu[b + 1];
  len = c1 - c0;
  start = padded ? (int64_t)b * max_seqlen : (int64_t)c0;
}

// Does row t belong to some sequence?
__device__ __forceinline__ bool row_in_sequence(int64_t t, const int* cu, int batch, int padded, int max_seqlen) {
  if (padded) {
    const int64_t b = t / max_seqlen;
    if (b >= batch) return false;
    return (t - b * max_seqlen) < (int64_t)(cu[b + 1] - cu[b]);
  }
  return t >= cu[0] && t < cu[batch];
}

// ------------------------------------------------------------------ buffer and tile helpers

// Row of a 32-row M-tile (Q, dO) that MFMA row m reads, and kv row of the 128-row tile that
// k-index k of the dQ GEMM reads. With rows padded by 16 bytes, this interleave makes the
// 16-byte operand reads (16 consecutive m) and the 4-row transpose reads (m = 4u..4u+3)
// touch distinct LDS banks.
__device__ __forceinline__ constexpr int tile_row(int m) { return ((m >> 2) & 3) + 4 * (m & 3) + 16 * (m >> 4); }

constexpr int kRsrcWord3 = 0x00020000;

// Buffer resource over [base, base + bytes): loads past the end return 0 and atomics past
// the end are dropped (raw buffer, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

// A buffer offset past every resource this file builds (the host keeps 128 rows of any tensor
// below 2^30 bytes): a load from it returns 0. Tile columns at or past a head dim that is smaller
// than the kernel's padded dim are read from here, so they hold zeros.
constexpr int kOutOfRange = 0x40000000;

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// 1 KB LDS-DMA transfers of a tile with padded rows of cpr 16-byte chunks: this lane's offset in
// transfer j. Chunks at or past the head dim d (zero columns up to the padded dim, row padding)
// read out of range and load zeros.
__device__ __forceinline__ int tile_dma_off(int j, int lane, int cpr, int row_bytes, int d) {
  const int p16 = 64 * j + lane;
  const int r = p16 / cpr, ch = p16 % cpr;
  return ch < d / 8 ? r * row_bytes + ch * 16 : kOutOfRange;
}

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// LDS-DMA of 16 bytes per lane: LDS[dst + 16 lane] = resource bytes [voff, voff + 16) (zeros past
// its end), like __builtin_amdgcn_raw_ptr_buffer_load_lds, but issued from an asm statement so that
// the compiler does not track it. The compiler cannot tell one LDS buffer from another, so after a
// tracked transfer it waits for every outstanding vector load before the next LDS read of any
// buffer, which stalls a pipeline that reads one buffer while the next one fills. The caller
// orders the transfer itself: s_waitcnt vmcnt(0) and a barrier before any read of the destination.
// The compiler's own waits stay correct beside it, since vector loads complete in issue order
// (the transfer only makes them wait longer). M0 holds the LDS address; the compiler writes M0
// before the statement, which starts with the wait state an LDS-DMA needs after that write.
__device__ __forceinline__ void dma16_untracked(__amdgpu_buffer_rsrc_t r, int voff,
                                                __attribute__((address_space(3))) void* dst) {
  const unsigned m0 = (unsigned)(uintptr_t)dst;
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(m0) : "memory");
}

// Rows [start, start + len) of a sequence, clamped to the rows that exist, so that
// every later row check is a single comparison against the length.
__device__ __forceinline__ int clamp_len(int64_t start, int len, int64_t total) {
  if (start < 0 || start >= total || len <= 0) return 0;
  return (int)((int64_t)len < total - start ? (int64_t)len : total - start);
}

__device__ __forceinline__ int imin(int x, int y) { return x < y ? x : y; }
__device__ __forceinline__ int imax(int x, int y) { return x > y ? x : y; }

// ------------------------------------------------------------------ stage 1: row statistics

struct PreArgs {
  const bf16* o;
  const bf16* dout;
  const float* m;  // row max, or the log-sum-exp when l is null
  const float* l;  // row sum, or null
  const int* cu_q;
  const int* cu_kv;
  float* lse2;    // [H][total_q]: m*log2(e) + log2(l)
  float* dvec;    // [H][total_q]: rowsum(O*dO)
  float* dq_acc;  // [H][total_q][d_qk], zeroed when not null
  bf16* dq;       // when not null: rows outside every sequence are zeroed
  bf16* dk;
  bf16* dv;
  int64_t total_q, total_kv;
  int H, Hk, batch, max_seqlen_q, max_seqlen_kv, padded;  // query heads, K/V heads
  int d_qk, d_v;  // head dims of Q, K (dQ, dK) and of V, O, dO (dV); multiples of 8
};

// Sum of v over aligned groups of N lanes (N a power of two up to 32), in every lane of the group:
// DPP adds within each 16-lane row (quad swaps, then the half-row and row mirrors), one lane
// exchange across the two rows of a 32-lane group.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                              0xF, 0xF, true));
  };
  if constexpr (N >= 2) v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (N >= 16) v += dpp(v, std::integral_constant<int, 0x140>{}); // row_mirror
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  return v;
}

// One thread per 8 features of a (token, head) row; TPR is a power of two >= max(d_qk, d_v) / 8.
// Block i takes 256 / TPR consecutive tokens of head i % H (heads fastest across blocks, so the
// blocks in flight read one contiguous range of tokens), which makes the statistics it writes
// into the head-major [H][T_q] arrays one contiguous run. EXACT: d_qk = d_v = 8 TPR.
// Every load a thread needs (O, dO, m, l and the sequence offsets of its row's zero fills) is
// issued before the first of them is used, so a wave waits for memory once.
template <int TPR, bool EXACT>
__global__ __launch_bounds__(256) void fa_bwd_pre(PreArgs a) {
  constexpr int RPB = 256 / TPR;  // tokens per block
  const int sub = threadIdx.x & (TPR - 1);
  const unsigned grp = blockIdx.x / (unsigned)a.H;
  const int h = (int)(blockIdx.x - grp * (unsigned)a.H);
  const int64_t t = (int64_t)grp * RPB + threadIdx.x / TPR;
  const int64_t pair = t * a.H + h;
  const int cq = EXACT ? TPR : a.d_qk / 8, cv = EXACT ? TPR : a.d_v / 8;  // 16-byte chunks per row
  const bool qrow = t < a.total_q;
  bf16x8 ov{}, gv{};
  if (qrow && sub < cv) {
    const int64_t off = pair * (8 * cv) + sub * 8;
    // read once: non-temporal, so that the streamed rows do not displace cached tiles
    ov = __builtin_nontemporal_load((const bf16x8*)(a.o + off));
    gv = __builtin_nontemporal_load((const bf16x8*)(a.dout + off));
  }
  float mv = 0.f, lv = 1.f;
  if (qrow && sub == 0) {
    mv = a.m[pair];
    if (a.l) lv = a.l[pair];
  }
  const bool zero_q = qrow && a.dq && sub < cq && !row_in_sequence(t, a.cu_q, a.batch, a.padded, a.max_seqlen_q);
  const bool zero_kv = h < a.Hk && t < a.total_kv && !row_in_sequence(t, a.cu_kv, a.batch, a.padded, a.max_seqlen_kv);
  const u32x4 z = {0u, 0u, 0u, 0u};
  if (qrow) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += from_bf16(ov[e]) * from_bf16(gv[e]);
    acc = group_sum<TPR>(acc);  // partners share the row
    if (a.dq_acc && sub < cq) {  // single-pass form: its fp32 dQ accumulator starts at 0
      float* accrow = a.dq_acc + ((int64_t)h * a.total_q + t) * (8 * cq) + sub * 8;
      const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
      *(f32x4*)accrow = zf;
      *(f32x4*)(accrow + 4) = zf;
    }
    if (zero_q) *(u32x4*)(a.dq + pair * (8 * cq) + sub * 8) = z;
    if (sub == 0) {
      const int64_t sidx = (int64_t)h * a.total_q + t;
      a.dvec[sidx] = acc;
      // (m, l) from the forward, or (when l is null) m holds the log-sum-exp m + ln(l) itself
      a.lse2[sidx] = a.l ? mv * kLog2e + __log2f(lv) : mv * kLog2e;
    }
  }
  if (zero_kv) {
    const int64_t kr = t * a.Hk + h;
    if (sub < cq) *(u32x4*)(a.dk + kr * (8 * cq) + sub * 8) = z;
    if (sub < cv) *(u32x4*)(a.dv + kr * (8 * cv) + sub * 8) = z;
  }
}

// ------------------------------------------------------------------ stage 2: single-pass main kernel

struct MainArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse2;
  const float* dvec;
  const int* cu_q;
  const int* cu_kv;
  float* dq_acc;  // fp32 [H][total_q][D] accumulator (single-pass form)
  bf16* dq;       // bf16 output (recompute form)
  bf16* dk;
  bf16* dv;
  int64_t total_q, total_kv;
  int H, Hk, batch, max_seqlen_q, max_seqlen_kv, padded, causal;  // query heads, K/V heads (H % Hk == 0)
  int window;        // > 0: each query sees only its left local window of keys (i - window, i]
  int d_qk, d_v;     // head dims of Q, K (dQ, dK) and of V, dO (dV): at most the kernel's padded dims
  float scale_log2;  // scale * log2(e)
  float scale;
  const int* sched;  // recompute kernels: (tile, sequence * heads + head) per workgroup, or null (dense grid)
  int head_major;    // recompute kernels, dense grid, (K/V) heads x sequences a multiple of 8: each XCD
                     // takes the tiles of one (sequence, head) at a time
  bf16* ds;          // stored-dS form: dS blocks of 32 q rows x 256 keys (64-key dK/dV kernel) or pieces of
                     // 32 q rows x 32 keys (wide-head kernels), [sequence][head][ds_nkt][ds_nqs]
  int ds_nqs, ds_nkt;  // 32-row q steps, and 256-key (blocks) or 32-key (pieces) kv tiles, of the longest
                       // sequences
};

// Stored-dS form of the wide-head kernels: one dS piece holds a 32-row q step against a 32-key tile,
// 2 KB of bf16 in the order a wave's lanes hold the values after the dK/dV kernel's softmax (half s2 of
// 1 KB holds, at lane c + 32 hh, the 16 bytes of dsk[s2]). Piece (t, kt) of (sequence b, query head h)
// starts at element ds_piece(b * H + h, kt, t).
constexpr int kDsPiece = 32 * 32;
__device__ __forceinline__ int64_t ds_piece(const MainArgs& a, int hb, int kt, int t) {
  return (((int64_t)hb * a.ds_nkt + kt) * a.ds_nqs + t) * kDsPiece;
}

// Splits of the split-and-reduce form: workgroups per (head, sequence), each with its own fp32 dQ
// buffer; split s takes the kv tiles s, s + kSplits, ...
constexpr int kSplits = 8;

template <int D>
struct MainCfg {
  static constexpr int BN = 128;                 // kv rows per workgroup (32 per wave)
  static constexpr int BM = 64;                  // q rows per step
  static constexpr int NW = 4;                   // waves
  static constexpr int KSD = D / 16;             // MFMA k-steps over the head dim
  static constexpr int NTD = D / 32;             // 32-wide output tiles over the head dim
  static constexpr int TPW = D / 64;             // dQ output tiles per wave
  static constexpr int QS = D + 8;               // row stride (elements) of the Q, dO and K tiles
  static constexpr int SS = BM + 8;              // row stride (elements) of dS^T
  static constexpr int CPR = QS / 8;             // 16-byte chunks per padded row
  static constexpr int TILE = BM * QS;           // elements of one Q or dO buffer
  static constexpr int TILE_BYTES = TILE * 2;
  static constexpr int NDMA = TILE_BYTES / 1024; // 1 KB LDS-DMA transfers per tile
  static constexpr int OFF_K = 0;                          // K tile [BN][QS]
  static constexpr int OFF_Q = OFF_K + BN * QS * 2;        // Q [2][BM][QS]
  static constexpr int OFF_DO = OFF_Q + 2 * TILE_BYTES;    // dO [2][BM][QS]
  static constexpr int OFF_DS = OFF_DO + 2 * TILE_BYTES;   // dS^T [BN][SS]
  static constexpr int OFF_ST = OFF_DS + BN * SS * 2;      // [2 buffers][lse2, D][BM] fp32
  static constexpr int LDS_BYTES = OFF_ST + 4 * BM * 4;
  static_assert(TILE_BYTES % 1024 == 0, "a tile is a whole number of 1 KB transfers");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// The single-pass form: one workgroup per (kv tile, head, sequence) forms the dK, dV and dQ
// contributions of every (q tile, kv tile) pair and adds the dQ partials to the fp32 accumulator
// with atomics. SPLIT: one workgroup per (split, head, sequence) walks the kv tiles split,
// split + kSplits, ... in order and adds its dQ partials into its own fp32 buffer of the split
// with plain loads and stores (the split's first tile stores); fa_bwd_split_reduce sums the splits.
template <int D, bool CAUSAL, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fa_bwd_main(MainArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using C = MainCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, QS = C::QS, SS = C::SS;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  bf16* s_k = (bf16*)(smem + C::OFF_K);
  bf16* s_q = (bf16*)(smem + C::OFF_Q);
  bf16* s_do = (bf16*)(smem + C::OFF_DO);
  bf16* s_dst = (bf16*)(smem + C::OFF_DS);
  float* s_st = (float*)(smem + C::OFF_ST);

  const int HB = a.H * a.batch;
  const int first = blockIdx.x / HB;  // the kv tile (heavy low tiles of every head first), or the split
  const int hb = blockIdx.x - first * HB;
  const int b = hb / a.H, h = hb - (hb / a.H) * a.H;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int64_t rs = (int64_t)a.H * D;  // elements between consecutive tokens
  const int rsb = (int)(rs * 2);        // bytes between consecutive tokens
  const bf16* qb = a.q + q_start * rs + (int64_t)h * D;
  const bf16* db = a.dout + q_start * rs + (int64_t)h * D;
  const float* lse_b = a.lse2 + (int64_t)h * a.total_q + q_start;
  const float* dd_b = a.dvec + (int64_t)h * a.total_q + q_start;
  // the fp32 dQ accumulator [H][total_q][D], or the split's buffer in [kSplits][H][total_q][D]
  float* dq_b = a.dq_acc + (((SPLIT ? (int64_t)first * a.H : 0) + h) * a.total_q + q_start) * D;

  for (int tile = first; tile * BN < Lk; tile += kSplits) {
  const bool first_tile = tile == first;  // split: the first tile stores its dQ partials, later ones add
  const int kv0 = tile * BN;
  const bf16* kb = a.k + (kv_start + kv0) * rs + (int64_t)h * D;
  const bf16* vb = a.v + (kv_start + kv0) * rs + (int64_t)h * D;

  // ---- K tile -> LDS (kept for the dQ GEMM); K, V B-operand fragments of S and dP -> registers
  const int kv_rows = imin(Lk - kv0, BN);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (int64_t)kv_rows * rsb);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (int64_t)kv_rows * rsb);
  for (int ch = tid; ch < BN * D / 8; ch += 256) {
    const int r = ch / (D / 8), col = (ch % (D / 8)) * 8;
    *(u32x4*)(s_k + r * QS + col) = buf_load16(rk, r * rsb + col * 2);
  }
  bf16x8 kf[C::KSD], vf[C::KSD];
#pragma unroll
  for (int ks = 0; ks < C::KSD; ++ks) {
    const int off = (32 * w + c) * rsb + (16 * ks + 8 * hh) * 2;
    kf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
    vf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
  }
  {  // zero both Q and dO buffers once: rows past the sequence then hold zeros or earlier valid rows
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < 4 * C::TILE_BYTES; o += 256 * 16) *(u32x4*)(smem + C::OFF_Q + o) = z;
  }
  __syncthreads();  // zero fill and K tile written before any LDS-DMA lands

  f32x16 accK[C::NTD], accV[C::NTD];
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt) {
    accK[nt] = f32x16{};
    accV[nt] = f32x16{};
  }

  const int n_qt = (Lq + BM - 1) / BM;
  int qt = CAUSAL ? kv0 / BM : 0;
  const int ntq = (w * C::TPW) >> 1;  // this wave's 32-wide feature slice of dQ
  const int jcol = kv0 + 32 * w + c;  // this lane's key row (sequence-local) in S and dP

  // LDS-DMA: transfer j lands lane L at tile byte 1024 j + 16 L = padded row (64 j + L) / CPR,
  // chunk (64 j + L) % CPR; the pad chunk re-reads chunk 0 of its row (never used).
  constexpr int NJ = (C::NDMA + C::NW - 1) / C::NW;
  int dma_off[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int p16 = 64 * (w + C::NW * jj) + lane;
    const int r = p16 / C::CPR, ch = p16 % C::CPR;
    dma_off[jj] = r * rsb + (ch < D / 8 ? ch : 0) * 16;
  }
  auto issue_tile = [&](int t, int bi) {
    const int i0 = t * BM;
    const int64_t bytes = (int64_t)imin(Lq - i0, BM) * rsb;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb + (int64_t)i0 * rs, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(db + (int64_t)i0 * rs, bytes);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = w + C::NW * jj;
      if (j < C::NDMA) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rq, (__attribute__((address_space(3))) void*)(smem + C::OFF_Q + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rd, (__attribute__((address_space(3))) void*)(smem + C::OFF_DO + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
      }
    }
  };
  // row statistics of q tile t in MFMA row order: threads 0..63 lse2, 64..127 D. Rows past the
  // sequence get lse2 = +inf, so their P (and dS) is exactly 0 without a mask.
  auto load_stats = [&](int t) -> float {
    const int mi = tid & (BM - 1);
    const int r = t * BM + 32 * (mi >> 5) + tile_row(mi & 31);
    if (tid >= 2 * BM) return 0.f;
    if (r >= Lq) return tid < BM ? __builtin_inff() : 0.f;
    return (tid < BM ? lse_b : dd_b)[r];
  };
  auto store_stats = [&](int bi, float v) {
    if (tid < 2 * BM) s_st[bi * 2 * BM + tid] = v;
  };

  // one q tile: steps 1-7 of the per-tile math for this wave's 32 keys. Keys past the sequence
  // need no mask: their K rows are zero in LDS (no dQ contribution) and their dK/dV rows are
  // never written. Only the causal predicate is applied.
  auto tile_step = [&](int bi, int i0) {
    const bf16* sq = s_q + bi * C::TILE;
    const bf16* sd = s_do + bi * C::TILE;
    const float* st = s_st + bi * 2 * BM;
    const int jrel = jcol - i0;  // causal: key j is visible from tile row r iff jrel <= r
    const int arow = tile_row(c) * QS + 8 * hh;
    const int brow = (hh + 4 * (gi >> 2)) * QS + 16 * (g & 1) + 4 * (gi & 3);
    // steps 1 and 3 for M-tile mt: S = Q K^T, dP = dO V^T  ([q 32] x [kv 32] per wave)
    auto sdp = [&](int mt, f32x16& s, f32x16& dp) {
      s = f32x16{};
      dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KSD; ++ks) {
        const bf16x8 qa = *(const bf16x8*)(sq + arow + 32 * mt * QS + 16 * ks);
        const bf16x8 da = *(const bf16x8*)(sd + arow + 32 * mt * QS + 16 * ks);
        s = mfma32x32x16(qa, kf[ks], s);
        dp = mfma32x32x16(da, vf[ks], dp);
      }
    };
    // steps 2 and 5 for M-tile mt: P = exp2(S*scale*log2e - lse2), dS = P (dP - D), both to bf16
    auto softmax_ds = [&](int mt, const f32x16& s, const f32x16& dp, bf16x8 (&pk)[2], bf16x8 (&dsk)[2]) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int mrow = 32 * mt + 8 * a4 + 4 * hh;  // MFMA row of bb = 0
        const f32x4 lse = *(const f32x4*)(st + mrow);
        const f32x4 dd = *(const f32x4*)(st + BM + mrow);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int j = 4 * a4 + bb;
          float p = fast_exp2(s[j] * a.scale_log2 - lse[bb]);
          if constexpr (CAUSAL) p = (jrel <= 32 * mt + tile_row(8 * a4 + 4 * hh + bb)) ? p : 0.f;
          const float ds = p * (dp[j] - dd[bb]);
          pk[j >> 3][j & 7] = to_bf16(p);
          dsk[j >> 3][j & 7] = to_bf16(ds);
        }
      }
    };
    // steps 7 and 6 for M-tile mt: dV += P^T dO, dK += dS^T Q (scale applied at write-back). The
    // k-index e of the A operand is MFMA row 16 s2 + 4 hh + e (e < 4) or 16 s2 + 8 + 4 hh + e - 4;
    // the transpose reads fetch the matching tile rows.
    auto dvdk = [&](int mt, const bf16x8 (&pk)[2], const bf16x8 (&dsk)[2]) {
#pragma unroll
      for (int nt = 0; nt < C::NTD; ++nt) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int o = brow + (32 * mt + 16 * s2) * QS + 32 * nt;
          const bf16x8 bdo = concat(lds_read_tr4(sd + o), lds_read_tr4(sd + o + 2 * QS));
          const bf16x8 bq = concat(lds_read_tr4(sq + o), lds_read_tr4(sq + o + 2 * QS));
          accV[nt] = mfma32x32x16(pk[s2], bdo, accV[nt]);
          accK[nt] = mfma32x32x16(dsk[s2], bq, accK[nt]);
        }
      }
    };
    // Software pipeline over the two M-tiles: the softmax of one M-tile runs on the VALU while
    // the matrix cores work on the other's GEMMs.
    f32x16 s0, dp0, s1, dp1;
    bf16x8 pk0[2], dsk0[2], pk1[2], dsk1[2];
    sdp(0, s0, dp0);
    sdp(1, s1, dp1);
    softmax_ds(0, s0, dp0, pk0, dsk0);
    dvdk(0, pk0, dsk0);
    softmax_ds(1, s1, dp1, pk1, dsk1);
    dvdk(1, pk1, dsk1);
    // interleave: [S/dP 0] [S/dP 1 | softmax 0] [dV/dK 0 | softmax 1] [dV/dK 1]
#pragma unroll
    for (int i = 0; i < C::KSD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
    }
#pragma unroll
    for (int i = 0; i < C::KSD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 112 / C::KSD, 0);  // softmax VALU
    }
#pragma unroll
    for (int i = 0; i < 2 * C::NTD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 112 / (2 * C::NTD), 0);
    }
#pragma unroll
    for (int i = 0; i < 2 * C::NTD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // dS^T to LDS (for the dQ GEMM): row = this lane's key, 4 consecutive MFMA rows per store
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const bf16x8 src = (mt == 0 ? dsk0 : dsk1)[a4 >> 1];
        const int o4 = 4 * (a4 & 1);
        const bf16x4 v4 = {src[o4], src[o4 + 1], src[o4 + 2], src[o4 + 3]};
        *(bf16x4*)(s_dst + (32 * w + c) * SS + 32 * mt + 8 * a4 + 4 * hh) = v4;
      }
    }
  };

  int buf = 0;
  if (qt < n_qt) {
    issue_tile(qt, 0);
    store_stats(0, load_stats(qt));
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  for (; qt < n_qt; ++qt, buf ^= 1) {
    const bool has_next = qt + 1 < n_qt;
    float st_next = 0.f;
    if (has_next) {
      issue_tile(qt + 1, buf ^ 1);
      st_next = load_stats(qt + 1);
    }
    const int i0 = qt * BM;
    tile_step(buf, i0);
    __syncthreads();  // dS^T complete
    if (has_next) store_stats(buf ^ 1, st_next);

    // step 8: dQ partial = dS K over this tile's 128 keys, added to the fp32 accumulator (atomics)
    // or to the split's buffer (plain loads and stores: this thread is the only writer of these
    // elements). k-index 16 ks + 8 hh + 4 half + e reads kv row 16 ks + 2 hh + half + 4 e.
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(dq_b + (int64_t)i0 * D, (int64_t)imin(Lq - i0, BM) * D * 4);
    const int krow = 2 * hh + 4 * (gi >> 2);
    const int tcol = 16 * (g & 1) + 4 * (gi & 3);
#pragma unroll
    for (int tt = 0; tt < C::TPW; ++tt) {
      const int mtq = (w * C::TPW + tt) & 1;
      f32x16 acc = f32x16{};
      auto elem_off = [&](int a4, int bb) {
        return (32 * mtq + tile_row(8 * a4 + 4 * hh + bb)) * D * 4 + (32 * ntq + c) * 4;
      };
      f32x16 prev = f32x16{};  // split, later tiles: the partial sums so far, loaded ahead of the MFMAs
      if (SPLIT && !first_tile) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
            prev[4 * a4 + bb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rq, elem_off(a4, bb), 0, 0));
        }
      }
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) {
        const int ra = (16 * ks + krow) * SS + 32 * mtq + tcol;
        const int rb = (16 * ks + krow) * QS + 32 * ntq + tcol;
        const bf16x8 af = concat(lds_read_tr4(s_dst + ra), lds_read_tr4(s_dst + ra + SS));
        const bf16x8 bk = concat(lds_read_tr4(s_k + rb), lds_read_tr4(s_k + rb + QS));
        acc = mfma32x32x16(af, bk, acc);
      }
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          if constexpr (SPLIT)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, prev[4 * a4 + bb] + acc[4 * a4 + bb]), rq,
                                                  elem_off(a4, bb), 0, 0);
          else
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[4 * a4 + bb], rq, elem_off(a4, bb), 0, 0);
        }
      }
    }
    // the next tile's LDS-DMA (issued before this tile's atomics) must land before the barrier
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(16 * C::TPW));
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  // write-back: dK = scale * accK, dV = accV, bf16, rows of this wave's keys
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int r = kv0 + 32 * w + 8 * a4 + 4 * hh + bb;
        if (r < Lk) {
          const int64_t o = (kv_start + r) * rs + (int64_t)h * D + 32 * nt + c;
          a.dk[o] = to_bf16(accK[nt][4 * a4 + bb] * a.scale);
          a.dv[o] = to_bf16(accV[nt][4 * a4 + bb]);
        }
      }
    }
  }
  if constexpr (!SPLIT) break;  // one kv tile per workgroup
  __syncthreads();              // LDS reads of this tile done before the next tile's K and zero fill
  }
#endif
}


// ------------------------------------------------------------------ stage 2a: dK and dV by recompute

// Tiling of the dK/dV kernel for padded head dims DQ (Q, K) and DV (V, dO), multiples of 32, and NMT
// 32-row M-tiles per q step. Up to 128: a 128-row kv tile; each wave holds the K rows of its 32 keys
// in registers (the first GEMM then reads only Q, dO and V from LDS), the V tile sits in LDS. With
// NMT = 2, eight waves (two per SIMD, one workgroup per CU): the two waves of a 32-key group split
// each 64-row q step. With NMT = 1, four waves (72 KB of LDS at d = 128, so two workgroups share a
// CU and their waves do not wait on each other's barriers): each wave takes whole 32-row q steps for
// its keys. Wider heads: one wave per
// SIMD (accumulators in the larger register budget of a single wave), a 64-row kv tile whose K and V
// fragments are held in registers, so that LDS holds only the Q and dO tiles; with NMT = 2 four waves
// whose row groups' two waves swap P and dS each step and split the output tiles, with NMT = 1 (where
// one wave holds both outputs' accumulators, head dims summing to at most 320) two waves, each with
// whole 32-row q steps and whole sums for its keys, two workgroups per CU.
template <int DQ, int DV, int NMT_ = 2>
struct DkdvCfg {
  static constexpr bool WIDE = DQ > 128 || DV > 128;
  static constexpr int NMT = NMT_;               // M-tiles per step
  static_assert(NMT == 1 || NMT == 2, "one or two M-tiles per step");
  static constexpr bool SWAP = WIDE && NMT == 2;  // the two waves of a row group swap P and dS
  static constexpr int WPE = WIDE ? 1 : 2;       // waves per SIMD
  static constexpr int BN = WIDE ? 64 : 128;     // kv rows per workgroup: row groups of 32
  static constexpr int BM = 32 * NMT;            // q rows per step: M-tiles of 32
  static constexpr int NG = BN / 32;             // row groups
  static constexpr int NW = NMT * NG;            // waves: row groups x M-tiles
  static constexpr int NT = 64 * NW;
  static constexpr int KSQ = DQ / 16, KSV = DV / 16, KSM = KSQ > KSV ? KSQ : KSV;  // MFMA k-steps
  static constexpr int NTQ = DQ / 32, NTV = DV / 32, NTM = NTQ > NTV ? NTQ : NTV;  // 32-wide tiles
  static constexpr int QSQ = DQ + 8, QSV = DV + 8;  // padded row strides of the LDS tiles
  static constexpr int CPRQ = QSQ / 8, CPRV = QSV / 8;
  // one Q (dO) tile, and its buffer rounded up to whole 1 KB transfers (the rows past the tile that
  // the last transfer covers read out of range and land as zeros in the padding)
  static constexpr int TQ_BYTES = (BM * QSQ * 2 + 1023) / 1024 * 1024;
  static constexpr int TD_BYTES = (BM * QSV * 2 + 1023) / 1024 * 1024;
  static constexpr int NDMA_Q = TQ_BYTES / 1024, NDMA_D = TD_BYTES / 1024;
  // K is held in registers by every wave (B-operand fragments of its 32 keys); heads up to 128 keep
  // the V tile of the workgroup in LDS, wider heads hold V in registers as well
  static constexpr int V_BYTES = WIDE ? 0 : BN * QSV * 2;
  static constexpr int NDMA_V = V_BYTES / 1024;
  static constexpr int OFF_V = 0;                             // V [BN][QSV]
  static constexpr int OFF_Q = OFF_V + V_BYTES;               // Q [2][BM][QSQ]
  static constexpr int OFF_DO = OFF_Q + 2 * TQ_BYTES;         // dO [2][BM][QSV]
  static constexpr int OFF_ST = OFF_DO + 2 * TD_BYTES;        // [2 buffers][lse2, D][BM] fp32
  // wide heads: the two waves of a row group split the second GEMMs' output tiles, as many each; the
  // M-tile 0 wave takes dV tiles [0, NTV - BY) and dK tiles [NTQ - BX, NTQ), the other the rest
  static constexpr int BX = SWAP && NTQ > NTV ? (NTQ - NTV) / 2 : 0;
  static constexpr int BY = SWAP && NTV > NTQ ? (NTV - NTQ) / 2 : 0;
  static constexpr bool BAL = BX > 0 || BY > 0;      // each wave needs both P and dS of both M-tiles
  static constexpr int NTW = SWAP ? (NTQ + NTV) / 2 : 1;  // output tiles per wave
  static constexpr int OFF_X = OFF_ST + 4 * BM * 4;  // wide: [wave][lane] 2 bf16x8 of P or dS (4: both)
  static constexpr int PART_BYTES = NMT == 2 && !WIDE ? NG * (NTQ + NTV) * 64 * 64 : 0;  // partial dK, then dV
  static constexpr int TILE_END = OFF_X + (SWAP ? NW * 64 * (BAL ? 64 : 32) : 0);
  // the end-of-kernel exchange of partial sums reuses the whole allocation
  static constexpr int LDS_BYTES = TILE_END > PART_BYTES ? TILE_END : PART_BYTES;
  static_assert(DQ % 32 == 0 && DV % 32 == 0 && DQ <= 256 && DV <= 256, "padded head dims");
  static_assert(TQ_BYTES % 1024 == 0 && TD_BYTES % 1024 == 0 && V_BYTES % 1024 == 0,
                "tiles are whole 1 KB transfers");
  static_assert(LDS_BYTES <= (NMT == 1 ? 80 : 160) * 1024, "LDS budget (two workgroups per CU, or one)");
};

// dK and dV of one (kv tile, K/V head, sequence). Row group r = w % NG owns kv rows 32 r .. 32 r + 31,
// and with NMT = 2 the two waves of a group each take one 32-row M-tile mt = w / NG of every 64-row q
// step (NMT = 1: one wave per group, 32-row q steps). Each wave forms S = Q K^T, dP = dO V^T, P and dS
// for its M-tile (steps 1-5). Heads up to 128, and wider heads with NMT = 1: each wave accumulates its
// partial dV += P^T dO and dK += dS^T Q over its M-tile's rows (steps 7, 6), so the waves of a step
// never wait for each other, and with NMT = 2 after the last step the two waves of a group combine
// their partial sums through LDS (the M-tile 0 wave finishes dV, the other dK). Wider heads with
// NMT = 2, where both accumulators of a wave would not fit its registers next to the K and V fragments:
// the waves of a group swap P and dS through LDS each step, and split the output tiles, each over
// both M-tiles (wide_tile). Wide heads without a window, when a.ds is set: each wave also stores its
// step's dS as a piece of the stored-dS form (ds_piece), non-temporal (read once, by the dQ pass), at the
// start of the next step, so that the stores complete before the step's closing wait for its transfers.
template <int DQ, int DV, bool CAUSAL, bool WINDOW, bool EXACT, int NMT>
__global__ __attribute__((amdgpu_flat_work_group_size(DkdvCfg<DQ, DV, NMT>::NT, DkdvCfg<DQ, DV, NMT>::NT),
                          amdgpu_waves_per_eu(DkdvCfg<DQ, DV, NMT>::WPE, DkdvCfg<DQ, DV, NMT>::WPE)))
void fa_bwd_dkdv(MainArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = DkdvCfg<DQ, DV, NMT>;
  constexpr int BN = C::BN, BM = C::BM, NG = C::NG, QSQ = C::QSQ, QSV = C::QSV;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const bf16* s_v = (const bf16*)(smem + C::OFF_V);
  bf16* s_q = (bf16*)(smem + C::OFF_Q);
  bf16* s_do = (bf16*)(smem + C::OFF_DO);
  float* s_st = (float*)(smem + C::OFF_ST);

  // the host schedule names each workgroup's (kv tile, sequence * Hk + K/V head); the dense grid
  // puts the heavy (low) kv tiles first, tile-major over the heads and sequences, or head-major per
  // XCD (workgroup i runs on XCD i % 8): XCD x takes the kv tiles of (sequence, K/V head) x, then
  // x + 8, ..., so that its workgroups stream the same Q and dO tiles
  const int HB = a.Hk * a.batch;
  int tile, hb;
  if (a.sched) {
    tile = a.sched[2 * blockIdx.x];
    hb = a.sched[2 * blockIdx.x + 1];
  } else if (a.head_major) {  // HB % 8 == 0 (host): a bijection of the grid
    const int n_kt_max = (a.max_seqlen_kv + BN - 1) / BN;
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int k = slot / n_kt_max;
    tile = slot - k * n_kt_max;
    hb = x + 8 * k;
  } else {
    tile = blockIdx.x / HB;
    hb = blockIdx.x - tile * HB;
  }
  const int b = hb / a.Hk, hk = hb - (hb / a.Hk) * a.Hk;  // sequence, K/V head
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int kv0 = tile * BN;
  if (kv0 >= Lk) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int grp = w % NG, mt = w / NG;  // kv row group; M-tile
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int dqk = EXACT ? DQ : a.d_qk, dvd = EXACT ? DV : a.d_v;  // EXACT: the padded dims
  const int64_t rsq = (int64_t)a.H * dqk, rsd = (int64_t)a.H * dvd;     // row strides of Q and dO
  const int rsqb = (int)(rsq * 2), rsdb = (int)(rsd * 2);
  const int64_t rskq = (int64_t)a.Hk * dqk, rskv = (int64_t)a.Hk * dvd;  // of K (dK) and V (dV)
  const int rskqb = (int)(rskq * 2), rskvb = (int)(rskv * 2);
  const int G = a.H / a.Hk;  // query heads sharing this K/V head: hk * G .. hk * G + G - 1

  {  // zero the tiles once: rows past the sequences then hold zeros or earlier valid rows
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < C::OFF_ST; o += C::NT * 16) *(u32x4*)(smem + o) = z;
  }
  __syncthreads();

  // the q steps: for each query head of the group, the q tiles that can see these keys (causal: from
  // the tile of the first key on); step st is q tile qt0 + st % nq of query head hk * G + st / nq
  const int n_qt = (Lq + BM - 1) / BM;
  const int qt0 = CAUSAL ? kv0 / BM : 0;
  // window: the last query that sees a key of this tile is kv0 + BN - 2 + window
  const int qt_end = WINDOW ? imin(n_qt, (kv0 + BN - 2 + a.window) / BM + 1) : n_qt;
  const int nq = qt_end > qt0 ? qt_end - qt0 : 0;
  const int n_steps = G * nq;
  auto step_head = [&](int st) { return hk * G + st / nq; };
  auto step_tile = [&](int st) { return qt0 + st % nq; };
  const int jcol = kv0 + 32 * grp + c;  // this lane's key row (sequence-local)

  const int kv_rows = imin(Lk - kv0, BN);
  const bf16* kbase = a.k + (kv_start + kv0) * rskq + (int64_t)hk * dqk;
  const bf16* vbase = a.v + (kv_start + kv0) * rskv + (int64_t)hk * dvd;
  // this lane's K row (and, for wide heads, V row) as B-operand fragments: key 32 grp + c, features
  // 16 ks + 8 hh .. + 7 (zeros at or past the head dim)
  bf16x8 kreg[C::KSQ], vreg[C::WIDE ? C::KSV : 1];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, (int64_t)kv_rows * rskqb);
    const int row = 32 * grp + c;
#pragma unroll
    for (int ks = 0; ks < C::KSQ; ++ks) {
      const int col = 16 * ks + 8 * hh;
      kreg[ks] = __builtin_bit_cast(bf16x8, buf_load16(rk, col < dqk ? row * rskqb + col * 2 : kOutOfRange));
    }
  }
  if constexpr (C::WIDE) {
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, (int64_t)kv_rows * rskvb);
    const int row = 32 * grp + c;
#pragma unroll
    for (int ks = 0; ks < C::KSV; ++ks) {
      const int col = 16 * ks + 8 * hh;
      vreg[ks] = __builtin_bit_cast(bf16x8, buf_load16(rv, col < dvd ? row * rskvb + col * 2 : kOutOfRange));
    }
  } else {  // the V tile, once
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, (int64_t)kv_rows * rskvb);
    for (int j = w; j < C::NDMA_V; j += C::NW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(smem + C::OFF_V + 1024 * j),
                                               16, tile_dma_off(j, lane, C::CPRV, rskvb, dvd), 0, 0, 0);
  }
  constexpr int NJQ = (C::NDMA_Q + C::NW - 1) / C::NW, NJD = (C::NDMA_D + C::NW - 1) / C::NW;
  int offq[NJQ], offd[NJD];
#pragma unroll
  for (int jj = 0; jj < NJQ; ++jj) offq[jj] = tile_dma_off(w + C::NW * jj, lane, C::CPRQ, rsqb, dqk);
#pragma unroll
  for (int jj = 0; jj < NJD; ++jj) offd[jj] = tile_dma_off(w + C::NW * jj, lane, C::CPRV, rsdb, dvd);
  auto issue_tile = [&](int st, int bi) {
    const int i0 = step_tile(st) * BM, hq = step_head(st);
    const int rows = imin(Lq - i0, BM);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + (q_start + i0) * rsq + (int64_t)hq * dqk, (int64_t)rows * rsqb);
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(a.dout + (q_start + i0) * rsd + (int64_t)hq * dvd, (int64_t)rows * rsdb);
    // untracked (dma16_untracked): the step's LDS reads of the other buffer must not wait for these
    // transfers; wait_tiles and the step's barrier order them before buffer bi is read
    auto dma_q = [&](int jj, int j) {
      dma16_untracked(rq, offq[jj], (__attribute__((address_space(3))) void*)(smem + C::OFF_Q + bi * C::TQ_BYTES + 1024 * j));
    };
    auto dma_d = [&](int jj, int j) {
      dma16_untracked(rd, offd[jj], (__attribute__((address_space(3))) void*)(smem + C::OFF_DO + bi * C::TD_BYTES + 1024 * j));
    };
#pragma unroll
    for (int jj = 0; jj < (NJQ > NJD ? NJQ : NJD); ++jj) {
      const int j = w + C::NW * jj;
      if constexpr (C::NDMA_Q == C::NDMA_D) {  // one test for both tiles
        if (j < C::NDMA_Q) {
          dma_q(jj, j);
          dma_d(jj, j);
        }
      } else {
        if (jj < NJQ && j < C::NDMA_Q) dma_q(jj, j);
        if (jj < NJD && j < C::NDMA_D) dma_d(jj, j);
      }
    }
  };
  // row statistics of a q step in MFMA row order: threads 0..63 lse2, 64..127 D; rows past the
  // sequence get lse2 = +inf, so their P (and dS) is exactly 0 without a mask
  auto load_stats = [&](int st) -> float {
    const int mi = tid & (BM - 1);
    const int r = step_tile(st) * BM + 32 * (mi >> 5) + tile_row(mi & 31);
    if (tid >= 2 * BM) return 0.f;
    if (r >= Lq) return tid < BM ? __builtin_inff() : 0.f;
    const int64_t sidx = (int64_t)step_head(st) * a.total_q + q_start + r;
    return (tid < BM ? a.lse2 : a.dvec)[sidx];
  };
  auto store_stats = [&](int bi, float v) {
    if (tid < 2 * BM) s_st[bi * 2 * BM + tid] = v;
  };

  // partial dV and dK / scale of rows 32 grp .. +31 over this M-tile; with the P/dS swap (wider heads,
  // NMT = 2), acc_w holds this wave's NTW output tiles of those rows over whole steps (wide_tile)
  f32x16 acc_v[C::SWAP ? 1 : C::NTV], acc_k[C::SWAP ? 1 : C::NTQ], acc_w[C::NTW];
#pragma unroll
  for (int nt = 0; nt < C::NTV; ++nt) acc_v[C::SWAP ? 0 : nt] = f32x16{};
#pragma unroll
  for (int nt = 0; nt < C::NTQ; ++nt) acc_k[C::SWAP ? 0 : nt] = f32x16{};
#pragma unroll
  for (int i = 0; i < C::NTW; ++i) acc_w[i] = f32x16{};
  // wide heads: output tile i of the M-tile m wave is dV tile nt (is_v) or dK tile nt (wave-uniform)
  auto wide_tile = [&](int m, int i, bool& is_v, int& nt) {
    if (m == 0) {
      is_v = i < C::NTV - C::BY;
      nt = is_v ? i : C::NTQ - C::BX + (i - (C::NTV - C::BY));
    } else {
      is_v = i >= C::NTQ - C::BX;
      nt = is_v ? C::NTV - C::BY + (i - (C::NTQ - C::BX)) : i;
    }
  };

  const int arowq = (32 * mt + tile_row(c)) * QSQ + 8 * hh;  // A rows: this M-tile's q rows
  const int arowd = (32 * mt + tile_row(c)) * QSV + 8 * hh;
  const int vrow = (32 * grp + c) * QSV + 8 * hh;
  const int browq = (hh + 4 * (gi >> 2)) * QSQ + 16 * (g & 1) + 4 * (gi & 3) + 32 * mt * QSQ;
  const int browd = (hh + 4 * (gi >> 2)) * QSV + 16 * (g & 1) + 4 * (gi & 3) + 32 * mt * QSV;
  auto tile_q = [&](int bi) { return (const bf16*)s_q + bi * (C::TQ_BYTES / 2); };
  auto tile_do = [&](int bi) { return (const bf16*)s_do + bi * (C::TD_BYTES / 2); };

  // steps 1 and 3 for this wave's M-tile: S = Q K^T, dP = dO V^T  ([q 32] x [kv 32]); operands
  // are read PF k-steps ahead into distinct registers, one scheduling fence per k-step
  auto gemm1 = [&](int bi, f32x16& s, f32x16& dp) {
    const bf16* sq = tile_q(bi);
    const bf16* sd = tile_do(bi);
    s = f32x16{};
    dp = f32x16{};
    constexpr int PF = 2;
    bf16x8 qa[C::KSQ], da[C::KSV], kb[C::KSQ], vb[C::KSV];
    auto ld = [&](int ks) {
      if (ks < C::KSQ) {
        qa[ks] = *(const bf16x8*)(sq + arowq + 16 * ks);
        kb[ks] = kreg[ks];
      }
      if (ks < C::KSV) {
        da[ks] = *(const bf16x8*)(sd + arowd + 16 * ks);
        if constexpr (C::WIDE)
          vb[ks] = vreg[ks];
        else
          vb[ks] = *(const bf16x8*)(s_v + vrow + 16 * ks);
      }
    };
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) ld(ks);
#pragma unroll
    for (int ks = 0; ks < C::KSM; ++ks) {
      if (ks + PF < C::KSM) ld(ks + PF);
      if (ks < C::KSQ) s = mfma32x32x16(qa[ks], kb[ks], s);
      if (ks < C::KSV) dp = mfma32x32x16(da[ks], vb[ks], dp);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // steps 2 and 5 of step sp: P = exp2(S*scale*log2e - lse2) (causal: 0 where key > query),
  // dS = P (dP - D), as bf16 A operands
  auto softmax = [&](int sp, int bi, const f32x16& s, const f32x16& dp, bf16x8* pk, bf16x8* dsk) {
    const int i0 = step_tile(sp) * BM;
    const float* st = s_st + bi * 2 * BM + 32 * mt;
    const int jrel = jcol - i0 - 32 * mt;  // key j visible from M-tile row r iff jrel <= r
    auto body = [&](auto masked) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 lse = *(const f32x4*)(st + 8 * a4 + 4 * hh);
        const f32x4 dd = *(const f32x4*)(st + BM + 8 * a4 + 4 * hh);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int j = 4 * a4 + bb;
          float p = fast_exp2(s[j] * a.scale_log2 - lse[bb]);
          if constexpr (decltype(masked)::value) {
            const int r = tile_row(8 * a4 + 4 * hh + bb);
            if constexpr (WINDOW)  // key j visible from query i iff 0 <= i - j < window: one unsigned compare
              p = (unsigned)(r - jrel) < (unsigned)a.window ? p : 0.f;
            else
              p = (jrel <= r) ? p : 0.f;
          }
          pk[j >> 3][j & 7] = to_bf16(p);
          dsk[j >> 3][j & 7] = to_bf16(p * (dp[j] - dd[bb]));
        }
      }
    };
    // every key of the group visible from every query of the M-tile: no element mask (wave-uniform)
    const int kmin = kv0 + 32 * grp, qmin = i0 + 32 * mt;
    const bool full = !CAUSAL || (kmin + 31 <= qmin && (!WINDOW || qmin + 31 - a.window < kmin));
    if (full)
      body(std::false_type{});
    else
      body(std::true_type{});
  };
  // steps 7 and 6 over this M-tile: dV += P^T dO, dK += dS^T Q. k-step s2: its k-index e is MFMA
  // row 16 s2 + 4 hh + e (e < 4) or 16 s2 + 8 + 4 hh + e - 4; the transpose reads fetch those rows.
  // B operands are read PF MFMAs ahead; the dV and dK MFMAs alternate (independent chains).
  auto gemm2 = [&](int bi, const bf16x8* pk, const bf16x8* dsk) {
    const bf16* sq = tile_q(bi);
    const bf16* sd = tile_do(bi);
    constexpr int NB = 2 * C::NTM, PF = 2;
    bf16x8 bd[NB], bq[NB];
    auto ld = [&](int i) {
      const int s2 = i / C::NTM, nt = i % C::NTM;
      if (nt < C::NTV) {
        const int o = browd + 16 * s2 * QSV + 32 * nt;
        bd[i] = concat(lds_read_tr4(sd + o), lds_read_tr4(sd + o + 2 * QSV));
      }
      if (nt < C::NTQ) {
        const int o = browq + 16 * s2 * QSQ + 32 * nt;
        bq[i] = concat(lds_read_tr4(sq + o), lds_read_tr4(sq + o + 2 * QSQ));
      }
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) ld(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i + PF < NB) ld(i + PF);
      const int s2 = i / C::NTM, nt = i % C::NTM;
      if (nt < C::NTV) acc_v[C::SWAP ? 0 : nt] = mfma32x32x16(pk[s2], bd[i], acc_v[C::SWAP ? 0 : nt]);
      if (nt < C::NTQ) acc_k[C::SWAP ? 0 : nt] = mfma32x32x16(dsk[s2], bq[i], acc_k[C::SWAP ? 0 : nt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the wide heads' step 7 / step 6 over the whole step: swap with the partner wave (the M-tile 0
  // wave needs the partner's P for dV, the other the partner's dS for dK), then one GEMM over the
  // step's 64 q rows, k-steps in row order. Built once per M-tile (mt_c, called under a wave-uniform
  // branch), so that the roles' choices of A operands, output tiles and B rows are made at compile
  // time rather than by per-element selects
  auto gemm2_swap = [&](auto mt_c, int bi, const bf16x8* pk, const bf16x8* dsk) {
    constexpr int mt = decltype(mt_c)::value;
    // the balanced layout publishes four values per lane, stored [wave][value][lane] so that each 16-byte
    // access of a wave is one contiguous 1 KB run (a 64-byte lane stride costs bank conflicts: -6 % on
    // the balanced pass); two values keep [wave][lane][value], measured as fast or slightly faster
    constexpr int NX = C::BAL ? 4 : 2;  // bf16x8 each wave publishes per lane
    bf16x8* xs = (bf16x8*)(smem + C::OFF_X);
    const int partner = grp + NG * (1 - mt);
    auto xat = [&](int wave, int k) -> bf16x8& { return xs[(wave * NX + k) * 64 + lane]; };
    if constexpr (C::BAL) {  // both waves need P and dS of both M-tiles
      xat(w, 0) = pk[0];
      xat(w, 1) = pk[1];
      xat(w, 2) = dsk[0];
      xat(w, 3) = dsk[1];
    } else {  // the M-tile 0 wave forms dV (needs P), the other dK (needs dS)
      xs[(w * 64 + lane) * NX] = mt == 0 ? dsk[0] : pk[0];
      xs[(w * 64 + lane) * NX + 1] = mt == 0 ? dsk[1] : pk[1];
    }
    __syncthreads();
    // A operands of k-step 2 u + s2 (M-tile u, its k-step s2): P (for dV tiles) and dS (for dK tiles)
    bf16x8 ap[4], ad[4];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 op_, od_;
      if constexpr (C::BAL) {
        op_ = xat(partner, s2);
        od_ = xat(partner, 2 + s2);
      } else {
        op_ = od_ = xs[(partner * 64 + lane) * NX + s2];
      }
      ap[s2] = mt == 0 ? pk[s2] : op_;
      ap[2 + s2] = mt == 0 ? op_ : pk[s2];
      ad[s2] = mt == 0 ? dsk[s2] : od_;
      ad[2 + s2] = mt == 0 ? od_ : dsk[s2];
    }
    // B: dO rows (for dV tiles) or Q rows (for dK tiles) of the step, read transposed
    const int browv = (hh + 4 * (gi >> 2)) * QSV + 16 * (g & 1) + 4 * (gi & 3);
    const int browk = (hh + 4 * (gi >> 2)) * QSQ + 16 * (g & 1) + 4 * (gi & 3);
    constexpr int NB = 4 * C::NTW, PF = 2;
    bf16x8 bw[NB];
    auto ld = [&](int i) {
      const int ksi = i / C::NTW;
      bool is_v;
      int nt;
      wide_tile(mt, i % C::NTW, is_v, nt);
      const int qs = is_v ? QSV : QSQ;
      const bf16* bsrc = is_v ? tile_do(bi) : tile_q(bi);
      const int o = (is_v ? browv : browk) + 16 * ksi * qs + 32 * nt;
      bw[i] = concat(lds_read_tr4(bsrc + o), lds_read_tr4(bsrc + o + 2 * qs));
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) ld(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i + PF < NB) ld(i + PF);
      const int ksi = i / C::NTW, t = i % C::NTW;
      bool is_v;
      int nt;
      wide_tile(mt, t, is_v, nt);
      acc_w[t] = mfma32x32x16(is_v ? ap[ksi] : ad[ksi], bw[i], acc_w[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto wait_tiles = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's LDS-DMA transfers and loads have landed
    __builtin_amdgcn_sched_barrier(0);
  };

  // all waves in step: tile sp + 1 loads while step sp runs; one barrier per step
  f32x16 s, dp;
  bf16x8 pk[2], dsk[2], dsk_prev[2];
  // this wave's stored-dS piece of step st: 32-row q step t, 32-key tile kt (wide heads, no window)
  constexpr bool kPieces = C::WIDE && !WINDOW;
  auto store_piece = [&](int st, const bf16x8 (&d)[2]) {
    if constexpr (kPieces) {
      if (a.ds) {
        const int t = step_tile(st) * C::NMT + mt, kt = tile * NG + grp;
        if (t < a.ds_nqs && kt < a.ds_nkt) {  // inside the workspace (lengths within the maxima)
          bf16* pc = a.ds + ds_piece(a, b * a.H + step_head(st), kt, t) + lane * 8;
          __builtin_nontemporal_store(d[0], (bf16x8*)pc);
          __builtin_nontemporal_store(d[1], (bf16x8*)(pc + 512));
        }
      }
    }
  };
  if (n_steps > 0) {
    issue_tile(0, 0);
    store_stats(0, load_stats(0));
  }
  wait_tiles();
  __syncthreads();
  if constexpr (C::SWAP) {
    // one copy of the loop per M-tile (a branch inside it would make the two gemm2_swap copies
    // keep the accumulators in different registers, and copy them back every step)
    auto step_loop = [&](auto mt_c) {
      for (int sp = 0, buf = 0; sp < n_steps; ++sp, buf ^= 1) {
        const bool has_next = sp + 1 < n_steps;
        float st_next = 0.f;
        if (has_next) {
          issue_tile(sp + 1, buf ^ 1);
          st_next = load_stats(sp + 1);
        }
        if (sp > 0) store_piece(sp - 1, dsk_prev);
        gemm1(buf, s, dp);
        softmax(sp, buf, s, dp, pk, dsk);
        if constexpr (kPieces) {
          dsk_prev[0] = dsk[0];
          dsk_prev[1] = dsk[1];
        }
        gemm2_swap(mt_c, buf, pk, dsk);
        if (has_next) store_stats(buf ^ 1, st_next);
        wait_tiles();
        __syncthreads();
      }
    };
    if (mt == 0)
      step_loop(std::integral_constant<int, 0>{});
    else
      step_loop(std::integral_constant<int, 1>{});
  } else {
    for (int sp = 0, buf = 0; sp < n_steps; ++sp, buf ^= 1) {
      const bool has_next = sp + 1 < n_steps;
      float st_next = 0.f;
      if (has_next) {
        issue_tile(sp + 1, buf ^ 1);
        st_next = load_stats(sp + 1);
      }
      if (sp > 0) store_piece(sp - 1, dsk_prev);
      gemm1(buf, s, dp);
      softmax(sp, buf, s, dp, pk, dsk);
      if constexpr (kPieces) {
        dsk_prev[0] = dsk[0];
        dsk_prev[1] = dsk[1];
      }
      gemm2(buf, pk, dsk);
      if (has_next) store_stats(buf ^ 1, st_next);
      wait_tiles();
      __syncthreads();
    }
  }
  if (n_steps > 0) store_piece(n_steps - 1, dsk_prev);  // the last step's piece

  // write-back of rows 32 grp .. 32 grp + 31, features below the head dim, in bf16
  auto store_dv = [&](const f32x16* acc) {
#pragma unroll
    for (int nt = 0; nt < C::NTV; ++nt) {
      if (32 * nt + c >= dvd) continue;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int r = kv0 + 32 * grp + 8 * a4 + 4 * hh + bb;
          if (r < Lk) a.dv[(kv_start + r) * rskv + (int64_t)hk * dvd + 32 * nt + c] = to_bf16(acc[nt][4 * a4 + bb]);
        }
      }
    }
  };
  auto store_dk = [&](const f32x16* acc) {  // dK = scale * acc
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
      if (32 * nt + c >= dqk) continue;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int r = kv0 + 32 * grp + 8 * a4 + 4 * hh + bb;
          if (r < Lk)
            a.dk[(kv_start + r) * rskq + (int64_t)hk * dqk + 32 * nt + c] = to_bf16(acc[nt][4 * a4 + bb] * a.scale);
        }
      }
    }
  };
  if constexpr (C::SWAP) {  // this wave's output tiles (wide_tile): dV, and dK = scale * acc
#pragma unroll
    for (int i = 0; i < C::NTW; ++i) {
      bool is_v;
      int nt;
      wide_tile(mt, i, is_v, nt);
      const int dcol = 32 * nt + c;
      if (dcol >= (is_v ? dvd : dqk)) continue;
      bf16* dst = is_v ? a.dv : a.dk;
      const int64_t rs = is_v ? rskv : rskq;
      const int64_t col = (int64_t)hk * (is_v ? dvd : dqk) + dcol;
      const float sc = is_v ? 1.f : a.scale;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int r = kv0 + 32 * grp + 8 * a4 + 4 * hh + bb;
          if (r < Lk) dst[(kv_start + r) * rs + col] = to_bf16(acc_w[i][4 * a4 + bb] * sc);
        }
      }
    }
  } else if constexpr (C::NMT == 1) {  // each wave holds the whole sums of its keys
    store_dv(acc_v);
    store_dk(acc_k);
  } else {
    // combine the two M-tiles' partial sums through LDS, laid out as [NG][NTQ] partial dK tiles, then
    // [NG][NTV] partial dV tiles, each as 4 quarters of 64 lanes x 16 bytes (lane-contiguous, so the
    // 16-byte accesses hit distinct banks): the M-tile 0 wave keeps dV and takes the partner's dV, the
    // M-tile 1 wave keeps dK and takes the partner's dK; each writes the half its partner needs
    f32x4* part_k = (f32x4*)(smem) + (size_t)grp * C::NTQ * 256 + lane;
    f32x4* part_v = (f32x4*)(smem) + (size_t)(NG * C::NTQ + grp * C::NTV) * 256 + lane;
    auto put = [&](f32x4* dst, const f32x16& x) {
      dst[0] = __builtin_shufflevector(x, x, 0, 1, 2, 3);
      dst[64] = __builtin_shufflevector(x, x, 4, 5, 6, 7);
      dst[128] = __builtin_shufflevector(x, x, 8, 9, 10, 11);
      dst[192] = __builtin_shufflevector(x, x, 12, 13, 14, 15);
    };
    auto add = [&](f32x16& x, const f32x4* src) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 y = src[64 * q4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q4 + e] += y[e];
      }
    };
    if (mt == 0) {
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) put(part_k + nt * 256, acc_k[nt]);
    } else {
#pragma unroll
      for (int nt = 0; nt < C::NTV; ++nt) put(part_v + nt * 256, acc_v[nt]);
    }
    __syncthreads();
    if (mt == 0) {
#pragma unroll
      for (int nt = 0; nt < C::NTV; ++nt) add(acc_v[nt], part_v + nt * 256);
      store_dv(acc_v);
    } else {
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) add(acc_k[nt], part_k + nt * 256);
      store_dk(acc_k);
    }
  }
#endif
}

// ------------------------------------------------------------------ stage 2b: dQ by recompute

// Tiling of the dQ kernel and of the forward for padded head dims DQ (Q, K) and DV (V, dO):
// four waves of 32 q rows, kv steps of 64 keys whose K and V tiles stream through LDS. Heads up
// to 128 run two waves per SIMD; wider heads one (the larger register budget holds Q, dO and the
// accumulators).
template <int DQ, int DV>
struct DqCfg {
  static constexpr bool WIDE = DQ > 128 || DV > 128;
  static constexpr int WPE = WIDE ? 1 : 2;       // waves per SIMD
  static constexpr int NW = 4;                   // waves, 32 q rows each
  static constexpr int NT = 64 * NW;
  static constexpr int BQ = 32 * NW;             // q rows per workgroup
  static constexpr int BK = 64;                  // kv rows per step
  static constexpr int KSQ = DQ / 16, KSV = DV / 16, KSM = KSQ > KSV ? KSQ : KSV;  // MFMA k-steps
  static constexpr int NTQ = DQ / 32, NTV = DV / 32;                                // 32-wide tiles
  static constexpr int QSQ = DQ + 8, QSV = DV + 8;  // padded row strides of the K and V tiles
  static constexpr int CPRQ = QSQ / 8, CPRV = QSV / 8;
  static constexpr int TK_BYTES = BK * QSQ * 2, TV_BYTES = BK * QSV * 2;
  static constexpr int NDMA_K = TK_BYTES / 1024, NDMA_V = TV_BYTES / 1024;
  static constexpr int OFF_K = 0;                          // K [2][BK][QSQ]
  static constexpr int OFF_V = OFF_K + 2 * TK_BYTES;       // V [2][BK][QSV]
  static constexpr int LDS_BYTES = OFF_V + 2 * TV_BYTES;
  static_assert(DQ % 32 == 0 && DV % 32 == 0 && DQ <= 256 && DV <= 256, "padded head dims");
  static_assert(TK_BYTES % 1024 == 0 && TV_BYTES % 1024 == 0, "a tile is a whole number of 1 KB transfers");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// The K and V tiles of kv step t into buffer bi (each wave issues transfers w, w + NW, ...).
template <class C>
struct KvTileLoader {
  static constexpr int NJK = (C::NDMA_K + C::NW - 1) / C::NW, NJV = (C::NDMA_V + C::NW - 1) / C::NW;
  int offk[NJK], offv[NJV];
  __device__ __forceinline__ KvTileLoader(int w, int lane, int rskqb, int rskvb, int dqk, int dvd) {
#pragma unroll
    for (int jj = 0; jj < NJK; ++jj) offk[jj] = tile_dma_off(w + C::NW * jj, lane, C::CPRQ, rskqb, dqk);
#pragma unroll
    for (int jj = 0; jj < NJV; ++jj) offv[jj] = tile_dma_off(w + C::NW * jj, lane, C::CPRV, rskvb, dvd);
  }
  // untracked transfers (dma16_untracked): the step's LDS reads of the other buffer must not wait for
  // them; the end-of-step wait and barrier order them before their buffer is read
  __device__ __forceinline__ void issue(char* smem, int w, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                        int bi) const {
    auto dma_k = [&](int jj, int j) {
      dma16_untracked(rk, offk[jj], (__attribute__((address_space(3))) void*)(smem + C::OFF_K + bi * C::TK_BYTES + 1024 * j));
    };
    auto dma_v = [&](int jj, int j) {
      dma16_untracked(rv, offv[jj], (__attribute__((address_space(3))) void*)(smem + C::OFF_V + bi * C::TV_BYTES + 1024 * j));
    };
#pragma unroll
    for (int jj = 0; jj < (NJK > NJV ? NJK : NJV); ++jj) {
      const int j = w + C::NW * jj;
      if constexpr (C::NDMA_K == C::NDMA_V) {  // one test for both tiles
        if (j < C::NDMA_K) {
          dma_k(jj, j);
          dma_v(jj, j);
        }
      } else {
        if (jj < NJK && j < C::NDMA_K) dma_k(jj, j);
        if (jj < NJV && j < C::NDMA_V) dma_v(jj, j);
      }
    }
  }
};

// dQ of one (q tile, head, sequence): loops over the kv tiles, recomputes S^T = K Q^T and
// dP^T = V dO^T with the forward's statistics (steps 1-5 of the per-tile math), and
// accumulates dQ^T = K^T dS^T (step 8) in registers; dQ is written once, in bf16.
// KS = 2 (heads up to 128): two groups of four waves per workgroup, each with its own K/V tile
// buffers; group g takes kv steps t0 + g, t0 + g + 2, ..., and at the end group 1's sums are added to
// group 0's through LDS (always in that order, so the result is deterministic). For grids with no
// more workgroups than CUs, where one group per workgroup leaves a single wave on each SIMD.
template <int DQ, int DV, bool CAUSAL, bool WINDOW, bool EXACT, int KS>
__global__ __attribute__((amdgpu_flat_work_group_size(DqCfg<DQ, DV>::NT * KS, DqCfg<DQ, DV>::NT * KS),
                          amdgpu_waves_per_eu(DqCfg<DQ, DV>::WPE, DqCfg<DQ, DV>::WPE)))
void fa_bwd_dq(MainArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = DqCfg<DQ, DV>;
  constexpr int BQ = C::BQ, BK = C::BK, QSQ = C::QSQ, QSV = C::QSV;
  static_assert(KS == 1 || (KS == 2 && !C::WIDE), "the key split needs two sets of tile buffers in LDS");
  static_assert(KS == 1 || C::NW * C::NTQ * 16 * 64 * 4 <= KS * C::LDS_BYTES, "the sums of group 1 fit the buffers");
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES * KS];

  // the host schedule names each workgroup's (q tile, sequence * H + head). The dense grid runs the q
  // tiles with the most keys (under a causal mask the last ones) first, tile-major over the heads and
  // sequences; or, head-major per XCD (workgroup i runs on XCD i % 8): XCD x takes the tiles of
  // (sequence, head) x, then x + 8, ..., so that its workgroups stream the same K and V tiles
  const int HB = a.H * a.batch;
  const int n_qt_max = (a.max_seqlen_q + BQ - 1) / BQ;
  int tr, hb;
  if (a.sched) {
    tr = 0;
    hb = a.sched[2 * blockIdx.x + 1];
  } else if (a.head_major) {  // HB % 8 == 0 (host): a bijection of the grid
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int k = slot / n_qt_max;
    tr = slot - k * n_qt_max;
    hb = x + 8 * k;
  } else {
    tr = blockIdx.x / HB;
    hb = blockIdx.x - tr * HB;
  }
  const int b = hb / a.H, h = hb - (hb / a.H) * a.H;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int qtile = a.sched ? a.sched[2 * blockIdx.x] : CAUSAL ? n_qt_max - 1 - tr : tr;
  const int i0 = qtile * BQ;
  if (i0 >= Lq) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int w = KS == 1 ? wv : wv & (C::NW - 1);            // the q wave: rows 32 w ..+31 of the tile
  const int gk = KS == 1 ? 0 : wv / C::NW;                  // the key group
  char* const gsm = smem + gk * C::LDS_BYTES;               // the group's K/V tile buffers
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int dqk = EXACT ? DQ : a.d_qk, dvd = EXACT ? DV : a.d_v;  // EXACT: the padded dims
  const int64_t rsq = (int64_t)a.H * dqk, rsd = (int64_t)a.H * dvd;     // row strides of Q (dQ) and dO
  const int rsqb = (int)(rsq * 2), rsdb = (int)(rsd * 2);
  const int64_t rskq = (int64_t)a.Hk * dqk, rskv = (int64_t)a.Hk * dvd;  // of K and V
  const int rskqb = (int)(rskq * 2), rskvb = (int)(rskv * 2);
  const int hk = h / (a.H / a.Hk);  // the K/V head this query head reads
  const bf16* kb = a.k + kv_start * rskq + (int64_t)hk * dqk;
  const bf16* vb = a.v + kv_start * rskv + (int64_t)hk * dvd;
  const bf16* qb = a.q + (q_start + i0) * rsq + (int64_t)h * dqk;
  const bf16* db = a.dout + (q_start + i0) * rsd + (int64_t)h * dvd;
  const int qi = i0 + 32 * w + c;  // this lane's query row (sequence-local) in S^T, dP^T and dQ^T

  // Q, dO as B operands of S^T = K Q^T and dP^T = V dO^T: row qi, features 16 ks + 8 hh ..+7
  // (zeros at or past the head dim)
  const int q_rows = imin(Lq - i0, BQ);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (int64_t)q_rows * rsqb);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(db, (int64_t)q_rows * rsdb);
  bf16x8 qf[C::KSQ], df[C::KSV];
#pragma unroll
  for (int ks = 0; ks < C::KSQ; ++ks) {
    const int col = 16 * ks + 8 * hh;
    qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, col < dqk ? (32 * w + c) * rsqb + col * 2 : kOutOfRange));
  }
#pragma unroll
  for (int ks = 0; ks < C::KSV; ++ks) {
    const int col = 16 * ks + 8 * hh;
    df[ks] = __builtin_bit_cast(bf16x8, buf_load16(rd, col < dvd ? (32 * w + c) * rsdb + col * 2 : kOutOfRange));
  }
  // rows past the sequence: lse2 = +inf makes P (and dS) exactly 0
  const float lse = qi < Lq ? a.lse2[(int64_t)h * a.total_q + q_start + qi] : __builtin_inff();
  const float dd = qi < Lq ? a.dvec[(int64_t)h * a.total_q + q_start + qi] : 0.f;

  int n_kt = (Lk + BK - 1) / BK;
  if (CAUSAL) n_kt = imin(n_kt, (i0 + BQ - 1) / BK + 1);
  // window: the first query of the tile sees no key before i0 - window + 1
  const int t0 = WINDOW ? imax(0, i0 - a.window + 1) / BK : 0;

  {  // zero the K and V buffers once (rows past the sequence are masked, but must be finite)
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < C::LDS_BYTES * KS; o += C::NT * KS * 16) *(u32x4*)(smem + o) = z;
  }
  __syncthreads();

  const KvTileLoader<C> loader(w, lane, rskqb, rskvb, dqk, dvd);
  auto issue_kv = [&](int t, int bi) {
    const int j0 = t * BK, rows = imin(Lk - j0, BK);
    loader.issue(gsm, w, make_rsrc(kb + (int64_t)j0 * rskq, (int64_t)rows * rskqb),
                 make_rsrc(vb + (int64_t)j0 * rskv, (int64_t)rows * rskvb), bi);
  };

  f32x16 acc[C::NTQ];
#pragma unroll
  for (int nt = 0; nt < C::NTQ; ++nt) acc[nt] = f32x16{};

  int buf = 0;
  if (n_kt > t0 + gk) issue_kv(t0 + gk, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  const int arowk = tile_row(c) * QSQ + 8 * hh;
  const int arowv = tile_row(c) * QSV + 8 * hh;
  const int browk = (hh + 4 * (gi >> 2)) * QSQ + 16 * (g & 1) + 4 * (gi & 3);
  // steps of both groups (the last one of group 1 may have no tile: it only keeps the barriers)
  const int n_it = (n_kt - t0 + KS - 1) / KS;
  for (int it = 0; it < n_it; ++it, buf ^= 1) {
    const int t = t0 + KS * it + gk;
    if (t + KS < n_kt) issue_kv(t + KS, buf ^ 1);
    if (KS == 1 || t < n_kt) {
      const bf16* sk = (const bf16*)(gsm + C::OFF_K + buf * C::TK_BYTES);
      const bf16* sv = (const bf16*)(gsm + C::OFF_V + buf * C::TV_BYTES);
      // steps 1 and 3, transposed: S^T = K Q^T and dP^T - D = V dO^T - D ([kv 64] x [q 32] per wave;
      // the dP accumulators start from -D of the lane's query row, which folds the subtraction of
      // step 5 into the GEMM)
      f32x16 s[2], dp[2];
      float ndd = -dd;
      asm volatile("" : "+v"(ndd));  // formed per step: a splat kept across the loop would spill
  #pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        s[mt] = f32x16{};
  #pragma unroll
        for (int j = 0; j < 16; ++j) dp[mt][j] = ndd;
      }
      {  // operands read PF k-steps ahead into distinct registers, one scheduling fence per k-step
        constexpr int PF = 2;
        bf16x8 ka[C::KSQ][2], va[C::KSV][2];
        auto ld = [&](int ks) {
  #pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            if (ks < C::KSQ) ka[ks][mt] = *(const bf16x8*)(sk + arowk + 32 * mt * QSQ + 16 * ks);
            if (ks < C::KSV) va[ks][mt] = *(const bf16x8*)(sv + arowv + 32 * mt * QSV + 16 * ks);
          }
        };
  #pragma unroll
        for (int ks = 0; ks < PF; ++ks) ld(ks);
  #pragma unroll
        for (int ks = 0; ks < C::KSM; ++ks) {
          if (ks + PF < C::KSM) ld(ks + PF);
  #pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            if (ks < C::KSQ) s[mt] = mfma32x32x16(ka[ks][mt], qf[ks], s[mt]);
            if (ks < C::KSV) dp[mt] = mfma32x32x16(va[ks][mt], df[ks], dp[mt]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // steps 2 and 5: P = exp2(S*scale*log2e - lse2), dS = P (dP - D); key row j = t*BK + kv row.
      // Visible iff j < Lk and (causal) j <= qi: one bound per lane on the tile-local kv row.
      const int lim = CAUSAL ? imin(Lk - 1, qi) - t * BK : Lk - 1 - t * BK;
      // window: visible iff lo <= kr <= lim, one unsigned compare of kr - lo against lim - lo (a row
      // that sees no key of the tile gets a base past every kv row)
      const int lo = qi - a.window + 1 - t * BK;
      const int wbase = lim >= lo ? lo : (1 << 30);
      const unsigned wspan = lim >= lo ? (unsigned)(lim - lo) : 0u;
      bf16x8 dsk[2][2];
      auto softmax = [&](auto masked) {
  #pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
  #pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
  #pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
              const int j = 4 * a4 + bb;
              float p = fast_exp2(s[mt][j] * a.scale_log2 - lse);
              if constexpr (decltype(masked)::value) {
                const int kr = 32 * mt + tile_row(8 * a4 + 4 * hh + bb);
                if constexpr (WINDOW)
                  p = (unsigned)(kr - wbase) <= wspan ? p : 0.f;
                else
                  p = kr <= lim ? p : 0.f;
              }
              dsk[mt][j >> 3][j & 7] = to_bf16(p * dp[mt][j]);
            }
          }
        }
      };
      // every key of the tile visible from every row of this wave: no element mask (wave-uniform)
      const int qmin = i0 + 32 * w, kmax = t * BK + BK - 1;
      const bool full = kmax <= Lk - 1 && (!CAUSAL || kmax <= qmin) && (!WINDOW || qmin + 31 - a.window < t * BK);
      if (full)
        softmax(std::false_type{});
      else
        softmax(std::true_type{});
      // step 8, transposed: dQ^T += K^T dS^T. k-step ksi = 2 mt + s2: its k-index e is kv MFMA row
      // 16 s2 + 4 hh + e (e < 4) or 16 s2 + 8 + 4 hh + e - 4 of M-tile mt; the transpose reads fetch
      // those K rows. k-steps run outside the NTQ independent accumulators; A operands are read PF
      // MFMAs ahead.
      {
        constexpr int NB = 4 * C::NTQ, PF = 3;
        bf16x8 kt[NB];
        auto kt_load = [&](int i) {
          const int ksi = i / C::NTQ, nt = i % C::NTQ;
          const int o = browk + 16 * ksi * QSQ + 32 * nt;
          return concat(lds_read_tr4(sk + o), lds_read_tr4(sk + o + 2 * QSQ));
        };
  #pragma unroll
        for (int i = 0; i < PF; ++i) kt[i] = kt_load(i);
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (i + PF < NB) kt[i + PF] = kt_load(i + PF);
          const int ksi = i / C::NTQ, nt = i % C::NTQ;
          acc[nt] = mfma32x32x16(kt[i], dsk[ksi >> 1][ksi & 1], acc[nt]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the next K/V tiles have landed
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  if constexpr (KS > 1) {  // group 1's sums through LDS (free after the loop's last barrier), added to group 0's
    float* red = (float*)smem + w * (C::NTQ * 16 * 64) + lane;
    if (gk == 1) {
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt)
#pragma unroll
        for (int j = 0; j < 16; ++j) red[(nt * 16 + j) * 64] = acc[nt][j];
    }
    __syncthreads();
    if (gk == 1) return;
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[nt][j] += red[(nt * 16 + j) * 64];
  }

  // dQ = scale * (dQ^T)^T in bf16: this lane holds features 32 nt + 8 a4 + 4 hh + bb of row qi
  if (qi < Lq) {
    bf16* dst = a.dq + (q_start + qi) * rsq + (int64_t)h * dqk + 4 * hh;
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        if (32 * nt + 8 * a4 + 4 * hh >= dqk) continue;  // head dims are multiples of 8
        const bf16x4 v4 = {to_bf16(acc[nt][4 * a4] * a.scale), to_bf16(acc[nt][4 * a4 + 1] * a.scale),
                           to_bf16(acc[nt][4 * a4 + 2] * a.scale), to_bf16(acc[nt][4 * a4 + 3] * a.scale)};
        *(bf16x4*)(dst + 32 * nt + 8 * a4) = v4;
      }
    }
  }
#endif
}

// ------------------------------------------------------------------ forward: O, m, l

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const int* cu_q;
  const int* cu_kv;
  bf16* o;   // [total_q][H][d_v]
  float* m;  // [total_q][H]: row max of the scaled visible logits
  float* l;  // [total_q][H]: row sum of exp(scaled logit - m) over visible keys
  int64_t total_q, total_kv;
  int H, Hk, batch, max_seqlen_q, max_seqlen_kv, padded;  // query heads, K/V heads (H % Hk == 0)
  int window;        // > 0: each query sees only its left local window of keys (i - window, i]
  int d_qk, d_v;     // head dims of Q, K and of V, O
  float scale_log2;  // scale * log2(e)
  const int* sched;  // (q tile, sequence * H + head) per workgroup, or null (dense grid)
};

// Rows outside every sequence: O = 0, m = 0, l = 1 (finite values a backward never reads).
// One thread per 8 features of an O row, 256 / TPR rows per block; TPR is a power of two >= d_v / 8.
template <int TPR>
__global__ __launch_bounds__(256) void fa_fwd_fill(FwdArgs a) {
  const int sub = threadIdx.x & (TPR - 1);
  const int64_t pair = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;  // = t * H + h
  const int64_t t = pair / a.H;
  if (t >= a.total_q || row_in_sequence(t, a.cu_q, a.batch, a.padded, a.max_seqlen_q)) return;
  const u32x4 z = {0u, 0u, 0u, 0u};
  if (sub < a.d_v / 8) *(u32x4*)(a.o + pair * a.d_v + sub * 8) = z;
  if (sub == 0) {
    a.m[pair] = 0.f;
    a.l[pair] = 1.f;
  }
}

// Forward of one (q tile, head, sequence), the producer of the backward's inputs: S^T = K Q^T on
// bf16 MFMA, softmax with a running row maximum (the forward that the per-tile backward math
// inverts: P = exp(S*scale - m) / l), O^T += V^T P^T in registers; O = O^T^T / l, m and l written
// once per row. Same tiling as the dQ kernel: Q in registers, K and V tiles of 64 keys streamed
// through LDS, each lane owns one query row (its MFMA column), so the running maximum, the row sum
// and the rescaling of its O row are per-lane values combined with the partner lane (lane ^ 32).
template <int DQ, int DV, bool CAUSAL, bool WINDOW, bool EXACT>
__global__ __attribute__((amdgpu_flat_work_group_size(DqCfg<DQ, DV>::NT, DqCfg<DQ, DV>::NT),
                          amdgpu_waves_per_eu(DqCfg<DQ, DV>::WPE, DqCfg<DQ, DV>::WPE)))
void fa_fwd(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = DqCfg<DQ, DV>;
  constexpr int BQ = C::BQ, BK = C::BK, QSQ = C::QSQ, QSV = C::QSV;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  // the host schedule names each workgroup's (q tile, sequence * H + head); in the dense grid under
  // a causal mask the q tiles with the most keys (the last ones) dispatch first
  const int HB = a.H * a.batch;
  const int tr = a.sched ? 0 : blockIdx.x / HB;
  const int hb = a.sched ? a.sched[2 * blockIdx.x + 1] : blockIdx.x - tr * HB;
  const int b = hb / a.H, h = hb - (hb / a.H) * a.H;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int n_qt_max = (a.max_seqlen_q + BQ - 1) / BQ;
  const int qtile = a.sched ? a.sched[2 * blockIdx.x] : CAUSAL ? n_qt_max - 1 - tr : tr;
  const int i0 = qtile * BQ;
  if (i0 >= Lq) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int dqk = EXACT ? DQ : a.d_qk, dvd = EXACT ? DV : a.d_v;  // EXACT: the padded dims
  const int64_t rsq = (int64_t)a.H * dqk, rso = (int64_t)a.H * dvd;     // row strides of Q and O
  const int rsqb = (int)(rsq * 2);
  const int64_t rskq = (int64_t)a.Hk * dqk, rskv = (int64_t)a.Hk * dvd;  // of K and V
  const int rskqb = (int)(rskq * 2), rskvb = (int)(rskv * 2);
  const int hk = h / (a.H / a.Hk);  // the K/V head this query head reads
  const bf16* kb = a.k + kv_start * rskq + (int64_t)hk * dqk;
  const bf16* vb = a.v + kv_start * rskv + (int64_t)hk * dvd;
  const bf16* qb = a.q + (q_start + i0) * rsq + (int64_t)h * dqk;
  const int qi = i0 + 32 * w + c;  // this lane's query row (sequence-local)

  const int q_rows = imin(Lq - i0, BQ);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (int64_t)q_rows * rsqb);
  bf16x8 qf[C::KSQ];
#pragma unroll
  for (int ks = 0; ks < C::KSQ; ++ks) {
    const int col = 16 * ks + 8 * hh;
    qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, col < dqk ? (32 * w + c) * rsqb + col * 2 : kOutOfRange));
  }

  int n_kt = (Lk + BK - 1) / BK;
  if (CAUSAL) n_kt = imin(n_kt, (i0 + BQ - 1) / BK + 1);
  // window: the first query of the tile sees no key before i0 - window + 1
  const int t0 = WINDOW ? imax(0, i0 - a.window + 1) / BK : 0;

  {  // zero the K and V buffers once (keys past the sequence are masked, but must be finite)
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < C::LDS_BYTES; o += C::NT * 16) *(u32x4*)(smem + o) = z;
  }
  __syncthreads();

  const KvTileLoader<C> loader(w, lane, rskqb, rskvb, dqk, dvd);
  auto issue_kv = [&](int t, int bi) {
    const int j0 = t * BK, rows = imin(Lk - j0, BK);
    loader.issue(smem, w, make_rsrc(kb + (int64_t)j0 * rskq, (int64_t)rows * rskqb),
                 make_rsrc(vb + (int64_t)j0 * rskv, (int64_t)rows * rskvb), bi);
  };

  f32x16 acc[C::NTV];  // O^T of this lane's row: features 32 nt + 8 a4 + 4 hh + bb
#pragma unroll
  for (int nt = 0; nt < C::NTV; ++nt) acc[nt] = f32x16{};
  float mrun = -__builtin_inff();  // running max of S*scale*log2(e) over the keys seen
  float lrun = 0.f;                // this lane's part of sum exp2(S*scale*log2(e) - mrun)

  int buf = 0;
  if (n_kt > t0) issue_kv(t0, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  const int arowk = tile_row(c) * QSQ + 8 * hh;
  const int browv = (hh + 4 * (gi >> 2)) * QSV + 16 * (g & 1) + 4 * (gi & 3);
  for (int t = t0; t < n_kt; ++t, buf ^= 1) {
    if (t + 1 < n_kt) issue_kv(t + 1, buf ^ 1);
    const bf16* sk = (const bf16*)(smem + C::OFF_K + buf * C::TK_BYTES);
    const bf16* sv = (const bf16*)(smem + C::OFF_V + buf * C::TV_BYTES);
    // S^T = K Q^T ([kv 64] x [q 32] per wave), operands read PF k-steps ahead
    f32x16 s[2] = {f32x16{}, f32x16{}};
    {
      constexpr int PF = 2;
      bf16x8 ka[C::KSQ][2];
      auto ld = [&](int ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) ka[ks][mt] = *(const bf16x8*)(sk + arowk + 32 * mt * QSQ + 16 * ks);
      };
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) ld(ks);
#pragma unroll
      for (int ks = 0; ks < C::KSQ; ++ks) {
        if (ks + PF < C::KSQ) ld(ks + PF);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) s[mt] = mfma32x32x16(ka[ks][mt], qf[ks], s[mt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // visible iff key j < Lk and (causal) j <= qi: one bound per lane on the tile-local key
    const int lim = CAUSAL ? imin(Lk - 1, qi) - t * BK : Lk - 1 - t * BK;
    const int lo = qi - a.window + 1 - t * BK;  // window: first visible tile-local key
    float x[2][16];
    float tmax = -__builtin_inff();
    auto scale_mask = [&](auto masked) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          x[mt][j] = s[mt][j] * a.scale_log2;
          if constexpr (decltype(masked)::value) {
            const int kr = 32 * mt + tile_row(8 * (j >> 2) + 4 * hh + (j & 3));
            x[mt][j] = (kr <= lim && (!WINDOW || kr >= lo)) ? x[mt][j] : -__builtin_inff();
          }
          tmax = fmaxf(tmax, x[mt][j]);
        }
      }
    };
    // every key of the tile visible from every row of this wave: no element mask (wave-uniform)
    const int qmin = i0 + 32 * w, kmax = t * BK + BK - 1;
    const bool full = kmax <= Lk - 1 && (!CAUSAL || kmax <= qmin) && (!WINDOW || qmin + 31 - a.window < t * BK);
    if (full)
      scale_mask(std::false_type{});
    else
      scale_mask(std::true_type{});
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(mrun, tmax);
    // no visible key yet: keep everything at zero (mnew = -inf would make exp2 produce NaN)
    const float mref = mnew == -__builtin_inff() ? 0.f : mnew;
    const float alpha = fast_exp2(mrun - mref);  // 0 while mrun = -inf
    mrun = mnew;
    bf16x8 pk[2][2];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(x[mt][j] - mref);
        psum += p;
        pk[mt][j >> 3][j & 7] = to_bf16(p);
      }
    }
    lrun = lrun * alpha + psum;
#pragma unroll
    for (int nt = 0; nt < C::NTV; ++nt) acc[nt] *= alpha;
    // O^T += V^T P^T: k-step ksi = 2 mt + s2, k-index e is key MFMA row 16 s2 + 4 hh + e (e < 4) or
    // 16 s2 + 8 + 4 hh + e - 4 of M-tile mt; the transpose reads fetch those V rows
    {
      constexpr int NB = 4 * C::NTV, PF = 3;
      bf16x8 vt[NB];
      auto vt_load = [&](int i) {
        const int ksi = i / C::NTV, nt = i % C::NTV;
        const int o = browv + 16 * ksi * QSV + 32 * nt;
        return concat(lds_read_tr4(sv + o), lds_read_tr4(sv + o + 2 * QSV));
      };
#pragma unroll
      for (int i = 0; i < PF; ++i) vt[i] = vt_load(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (i + PF < NB) vt[i + PF] = vt_load(i + PF);
        const int ksi = i / C::NTV, nt = i % C::NTV;
        acc[nt] = mfma32x32x16(vt[i], pk[ksi >> 1][ksi & 1], acc[nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the next K/V tiles have landed
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  const float lsum = lrun + __shfl_xor(lrun, 32);
  if (qi < Lq) {
    const bool any = mrun != -__builtin_inff();  // a valid row without keys: O = 0, m = 0, l = 1
    const float inv = any ? 1.f / lsum : 0.f;
    bf16* dst = a.o + (q_start + qi) * rso + (int64_t)h * dvd + 4 * hh;
#pragma unroll
    for (int nt = 0; nt < C::NTV; ++nt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        if (32 * nt + 8 * a4 + 4 * hh >= dvd) continue;  // head dims are multiples of 8
        const bf16x4 v4 = {to_bf16(acc[nt][4 * a4] * inv), to_bf16(acc[nt][4 * a4 + 1] * inv),
                           to_bf16(acc[nt][4 * a4 + 2] * inv), to_bf16(acc[nt][4 * a4 + 3] * inv)};
        *(bf16x4*)(dst + 32 * nt + 8 * a4) = v4;
      }
    }
    if (hh == 0) {
      const int64_t idx = (q_start + qi) * a.H + h;
      a.m[idx] = any ? mrun * (1.f / kLog2e) : 0.f;
      a.l[idx] = any ? lsum : 1.f;
    }
  }
#endif
}

// ------------------------------------------------------------------ stage 3: split-and-reduce dQ sum

// dQ = scale * (sum of the split buffers that hold each row, in split order), in bf16. Split s holds
// the rows its first kv tile (s * BN) reaches: all rows of the sequence, or under a causal mask the
// rows from s * BN on; a split without kv tiles holds none. One workgroup per (64-row block, head,
// sequence); rows outside every sequence are zeroed by fa_bwd_pre.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_split_reduce(MainArgs a) {
  constexpr int R = 64, CH = D / 8, BN = MainCfg<D>::BN;
  const int HB = a.H * a.batch;
  const int blk = blockIdx.x / HB;
  const int hb = blockIdx.x - blk * HB;
  const int b = hb / a.H, h = hb - (hb / a.H) * a.H;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int r0 = blk * R;
  if (r0 >= Lq) return;
  const int n_split = imin(kSplits, (Lk + BN - 1) / BN);  // splits with at least one kv tile
  const int64_t plane = (int64_t)a.H * a.total_q * D;       // one split's buffer
  const float* src0 = a.dq_acc + ((int64_t)h * a.total_q + q_start) * D;
  for (int idx = threadIdx.x; idx < R * CH; idx += 256) {
    const int r = r0 + idx / CH, ch = idx % CH;
    if (r >= Lq) continue;
    const int ns = a.causal ? imin(n_split, r / BN + 1) : n_split;
    // all kSplits loads in flight at once: splits past ns re-read the last one held (or split 0,
    // allocated but unused when no split holds the row) and are not added
    const int last = imax(ns - 1, 0);
    f32x4 vlo[kSplits], vhi[kSplits];
#pragma unroll
    for (int sp = 0; sp < kSplits; ++sp) {
      const float* src = src0 + imin(sp, last) * plane + (int64_t)r * D + ch * 8;
      vlo[sp] = *(const f32x4*)src;
      vhi[sp] = *(const f32x4*)(src + 4);
    }
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < kSplits; ++sp) {  // split order, the same for every run
      if (sp < ns) {
        lo += vlo[sp];
        hi += vhi[sp];
      }
    }
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[e] = to_bf16(lo[e] * a.scale);
      out[e + 4] = to_bf16(hi[e] * a.scale);
    }
    *(bf16x8*)(a.dq + (q_start + r) * ((int64_t)a.H * D) + (int64_t)h * D + ch * 8) = out;
  }
}

// ------------------------------------------------------------------ stage 3: single-pass dQ cast

template <int D>
__global__ __launch_bounds__(256) void fa_bwd_dq_cast(const float* dq_acc, bf16* dq, int64_t total_q, int H,
                                                      float scale) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int sub = threadIdx.x % TPR;
  const int64_t pair = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;  // = t * H + h
  const int64_t t = pair / H;
  if (t >= total_q) return;
  const int h = (int)(pair - t * H);
  const float* src = dq_acc + ((int64_t)h * total_q + t) * D + sub * 8;
  const f32x4 x0 = *(const f32x4*)src;
  const f32x4 x1 = *(const f32x4*)(src + 4);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = to_bf16(x0[e] * scale);
    r[e + 4] = to_bf16(x1[e] * scale);
  }
  *(bf16x8*)(dq + pair * D + sub * 8) = r;
}

}  // namespace fa
