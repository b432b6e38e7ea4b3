// fa_bwd.hip -- C ABI of the single-pass attention backward (include/fa_bwd.h):
// host-side validation, the handle's device workspace and the three launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <new>
#include <vector>

#include "fa_bwd.h"
#include "fa_bwd_dkdv64.hpp"
#include "fa_bwd_dqds.hpp"
#include "fa_bwd_launch.hpp"

struct fa_bwd_handle {
  fa_bwd_desc desc;
  bool single_pass;  // the single-pass main kernel: FA_BWD_ALGO_SINGLE_PASS or FA_BWD_ALGO_SPLIT_REDUCE
  bool split;        // FA_BWD_ALGO_SPLIT_REDUCE: dQ partials per split, then fa_bwd_split_reduce
  int device;
  float* dq_acc;  // [H][total_q][head_dim] (atomics) or [kSplits][H][total_q][head_dim] (split)
  float* lse2;    // [H][total_q]
  float* dvec;    // [H][total_q]
  bool profiling;
  std::vector<hipEvent_t> events;  // 4 per recorded run
  int64_t recorded;                // runs whose events are in `events`
  // host schedule (fa_bwd_plan): (tile, sequence * heads + head) pairs, the dK/dV kernel's items
  // first, then the dQ kernel's (also the forward's); null when there is no plan
  int32_t* sched;
  int64_t n_kv_items, n_q_items;
  int32_t plan_mask;
  // layout of the dK/dV kernel for heads up to 128: forced by the algorithm code, or chosen by load
  // balance (four_waves_balances) from the descriptor, without and with a causal bound; planned and
  // dense runs of a handle take the same layout, so that they agree bitwise
  int32_t dkdv_layout;  // 0: chosen, 1: eight waves, 2: four waves, 3: 64 keys per wave
  bool four_dense[2];
  int32_t layout[2];    // the layout (1, 2 or 3) runs without and with a causal bound take
  // the dQ and dK/dV kernels' dense grids in head-major order per XCD (head_major_balances), without
  // and with a causal bound
  bool dq_head_major[2], dkdv_head_major[2];
  // the stored-dS pass's dense grid in head-major order (two workgroups per CU at every head dim)
  bool ds_head_major[2];
  // the dQ kernel in two key groups per workgroup (dq_key_split)
  bool dq_split;
  // stored-dS form: the dK/dV kernel writes dS, and the dQ pass reads it, in the format ds_fmt gives for
  // runs without and with a causal bound (kDsNone, kDsBlocks: the 64-key kernel's 32 x 256 blocks,
  // kDsPieces: the wide-head kernel's 32 x 32 pieces); ds_form: some run takes it
  bool ds_form;
  int32_t ds_fmt[2];
  fa::bf16* ds;
  int32_t ds_nqs, ds_nkt_blocks, ds_nkt_pieces;
};

namespace {

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

constexpr int64_t kMaxGrid = 0x7fffffff;
constexpr int64_t kMaxProfiledRuns = 4096;

void release_events(fa_bwd_handle* h) {
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  h->events.clear();
  h->recorded = 0;
}

bool head_dim_ok(int32_t d) { return d >= 8 && d <= 256 && d % 8 == 0; }

// Work of the dK/dV workgroups of one sequence (lq queries, lk keys): the 64-row q steps each 128-row
// kv tile visits, bounded as the kernel bounds its loop (causal start, window band); adds the sum
// over the tiles to total and keeps the largest.
void dkdv_work(int64_t lq, int64_t lk, bool causal, int64_t w, int64_t& total, int64_t& largest, int64_t bn = 128,
               int64_t bm = 64) {
  const int64_t n_qs = (lq + bm - 1) / bm;
  for (int64_t kv0 = 0; kv0 < lk; kv0 += bn) {
    const int64_t qt0 = causal ? kv0 / bm : 0;
    const int64_t qt_end = w > 0 ? std::min(n_qs, (kv0 + bn - 2 + w) / bm + 1) : n_qs;
    const int64_t work = std::max<int64_t>(0, qt_end - qt0);
    total += work;
    largest = std::max(largest, work);
  }
}

// The four-wave dK/dV layout runs two workgroups per CU, each at about half the rate of one
// eight-wave workgroup. Longest-first dispatch then balances only while the largest workgroup,
// doubled, still fits within the average work per CU; otherwise the eight-wave layout is kept.
// (in double: with the largest descriptors the products pass the int64 range)
bool four_waves_balances(double total, double largest, int cus) { return 2.0 * largest * cus <= total; }

// Work of the dQ kernel's workgroups of one sequence: the 64-key steps each 128-row q tile visits,
// bounded as the kernel bounds its loop (causal end, window start).
void dq_work(int64_t lq, int64_t lk, bool causal, int64_t w, int64_t& total, int64_t& largest) {
  for (int64_t i0 = 0; i0 < lq; i0 += 128) {
    int64_t n_kt = (lk + 63) / 64;
    if (causal) n_kt = std::min(n_kt, (i0 + 127) / 64 + 1);
    const int64_t t0 = w > 0 ? std::max<int64_t>(0, i0 - w + 1) / 64 : 0;
    const int64_t work = std::max<int64_t>(0, n_kt - t0);
    total += work;
    largest = std::max(largest, work);
  }
}

// Head-major order per XCD (each of the 8 XCDs takes the tiles of one (sequence, head) at a time, so
// that its workgroups share the other side's tiles in L2) starts the last head's heaviest tiles late;
// it is taken when the heads x sequences divide over the XCDs and the largest workgroup is at most a
// quarter of the work per workgroup slot, where that lateness costs little.
bool head_major_balances(double total, double largest, int64_t slots, int64_t heads_x_seqs) {
  return heads_x_seqs % 8 == 0 && 4.0 * largest * slots <= total;
}

// The dQ kernel for heads up to 128 (narrow) runs two workgroups of four waves per CU, each wave over
// one 32-row q step. Where its dense grid has no more workgroups than CUs, that leaves at most one wave
// per SIMD with nothing to hide its waits behind; there it takes two key groups per workgroup (eight
// waves, one workgroup per CU), each over every other kv step.
bool dq_key_split(const fa_bwd_desc& d, bool narrow, int cus) {
  const int64_t q_blocks = (int64_t)((d.max_seqlen_q + 127) / 128) * d.num_heads * d.batch;
  return narrow && q_blocks <= cus;
}

// threads per (token, head) row of the row kernels: a power of two covering the wider row in
// 8-element chunks
int threads_per_row(int d_qk, int d_v) {
  const int chunks = (d_qk > d_v ? d_qk : d_v) / 8;
  int t = 1;
  while (t < chunks) t *= 2;
  return t;
}

// The stored-dS form of the wide-head kernels (a head dim above 128, no window) stores 32 x 32 pieces;
// at head dims of exactly 128 the form runs on the 64-key layout, which stores 32 x 256 blocks.
constexpr int32_t kDsNone = 0, kDsBlocks = 1, kDsPieces = 2;
bool ds_pieces_apply(const fa_bwd_desc& d) {
  const int32_t dv = d.head_dim_v == 0 ? d.head_dim : d.head_dim_v;
  return (d.head_dim > 128 || dv > 128) && d.window == 0;
}

// Bytes of the stored-dS form's workspace per (sequence, query head): 16 KiB blocks of (32-row q step) x
// (256-key kv tile), or 2 KiB pieces of (32-row q step) x (32-key tile); -1 when the size passes
// kDsMaxBytes (computed in double, so that no product overflows).
constexpr int64_t kDsMaxBytes = int64_t(1) << 47;
int64_t ds_bytes_of(const fa_bwd_desc& d, bool pieces, int32_t& nqs, int32_t& nkt) {
  const int kt = pieces ? 32 : 256;
  nqs = (d.max_seqlen_q + 31) / 32;
  nkt = (d.max_seqlen_kv + kt - 1) / kt;
  const double bytes = (double)nqs * nkt * d.num_heads * d.batch * (kt * 32.0 * 2);
  return bytes > (double)kDsMaxBytes ? -1 : (int64_t)bytes;
}

fa_bwd_status check_desc(const fa_bwd_desc* d) {
  if (!d) return FA_BWD_ERR_INVALID_ARGUMENT;
  if (d->batch < 1 || d->num_heads < 1 || d->max_seqlen_q < 1 || d->max_seqlen_kv < 1 || d->total_q < 1 ||
      d->total_kv < 1)
    return FA_BWD_ERR_INVALID_ARGUMENT;
  const int32_t dv = d->head_dim_v == 0 ? d->head_dim : d->head_dim_v;
  if (!head_dim_ok(d->head_dim) || !head_dim_ok(dv)) return FA_BWD_ERR_UNSUPPORTED;
  if (d->algorithm < FA_BWD_ALGO_DEFAULT || d->algorithm > FA_BWD_ALGO_STORED_DS) return FA_BWD_ERR_INVALID_ARGUMENT;
  const bool single = d->algorithm == FA_BWD_ALGO_SINGLE_PASS || d->algorithm == FA_BWD_ALGO_SPLIT_REDUCE;
  // the single-pass kernels exist for equal head dims of 64 and 128
  if (single && (dv != d->head_dim || (d->head_dim != 64 && d->head_dim != 128))) return FA_BWD_ERR_UNSUPPORTED;
  const int32_t hkv = d->num_heads_kv == 0 ? d->num_heads : d->num_heads_kv;
  if (hkv < 1 || d->num_heads % hkv != 0) return FA_BWD_ERR_INVALID_ARGUMENT;
  // the single-pass form owns one (kv tile, head) per workgroup; grouped K/V heads need the recompute form
  if (single && hkv != d->num_heads) return FA_BWD_ERR_UNSUPPORTED;
  if (d->window < 0) return FA_BWD_ERR_INVALID_ARGUMENT;
  // sequence positions, and a window clamped to max_seqlen_q, stay below 2^30: the kernels' tile and
  // window bounds (kv0 + tile + window, i - window - kv0) then fit in 32 bits
  if (d->max_seqlen_q > (1 << 30) || d->max_seqlen_kv > (1 << 30)) return FA_BWD_ERR_INVALID_ARGUMENT;
  if (single && d->window > 0) return FA_BWD_ERR_UNSUPPORTED;
  // the 64-key dK/dV layout exists for head dims of 128; the stored-dS form runs on it, or on the
  // wide-head kernels (a head dim above 128) without a window
  const bool d128 = d->head_dim == 128 && dv == 128;
  if (d->algorithm == FA_BWD_ALGO_RECOMPUTE_DQ_64K && !d128) return FA_BWD_ERR_UNSUPPORTED;
  if (d->algorithm == FA_BWD_ALGO_STORED_DS) {
    if (!d128 && !ds_pieces_apply(*d)) return FA_BWD_ERR_UNSUPPORTED;
    int32_t nqs, nkt;  // its dS workspace must have a size (at most 2^47 bytes)
    if (ds_bytes_of(*d, !d128, nqs, nkt) < 0) return FA_BWD_ERR_UNSUPPORTED;
  }
  // index arithmetic stays in int64; grids must fit the launch limits
  const int64_t rows = (d->total_q > d->total_kv ? d->total_q : d->total_kv);
  if (rows > (int64_t(1) << 40) / d->num_heads) return FA_BWD_ERR_INVALID_ARGUMENT;
  // 128 rows of any tensor span less than 2^30 bytes: the kernels' 32-bit tile offsets, and the
  // out-of-range offset that reads zeros, rely on it
  const int64_t dmax = d->head_dim > dv ? d->head_dim : dv;
  if ((int64_t)d->num_heads * dmax * 2 * 128 >= (int64_t(1) << 30)) return FA_BWD_ERR_INVALID_ARGUMENT;
  const int64_t kv_tiles = (d->max_seqlen_kv + 63) / 64;  // the smallest kv tile of any kernel
  if (kv_tiles * d->num_heads * d->batch > kMaxGrid) return FA_BWD_ERR_INVALID_ARGUMENT;
  const int64_t q_tiles = (d->max_seqlen_q + 63) / 64;  // the split reduce's 64-row blocks
  if (q_tiles * d->num_heads * d->batch > kMaxGrid) return FA_BWD_ERR_INVALID_ARGUMENT;
  if (d->algorithm == FA_BWD_ALGO_SPLIT_REDUCE && (int64_t)fa::kSplits * d->num_heads * d->batch > kMaxGrid)
    return FA_BWD_ERR_INVALID_ARGUMENT;
  const int64_t rows_per_block = 256 / threads_per_row(d->head_dim, dv);
  // the row kernels: one block per (group of rows_per_block tokens, head), or per rows_per_block rows
  if ((rows + rows_per_block - 1) / rows_per_block * d->num_heads > kMaxGrid ||
      (rows * d->num_heads + rows_per_block - 1) / rows_per_block > kMaxGrid)
    return FA_BWD_ERR_INVALID_ARGUMENT;
  return FA_BWD_OK;
}

// The dK/dV kernel with 64 keys per wave: head dims of exactly 128 (with or without a window).
bool keys64_applies(const fa_bwd_desc& d) { return d.head_dim == 128 && d.head_dim_v == 128; }

// The 64-key dK/dV layout runs one workgroup per CU over 256 keys (and every query head of its K/V
// head): the default takes it where longest-first dispatch balances, i.e. the largest workgroup,
// doubled, fits within the average work per CU. Small grids, and grouped K/V heads that multiply each
// workgroup's work, keep the 128-key layouts; so do windows, whose band edges put the element mask on
// a large share of the 64-key kernel's steps (the four-wave layout measured faster there).
bool keys64_balances(double total, double largest, int cus) { return 2.0 * largest * cus <= total; }

void launch_dkdv64(const fa::MainArgs& ma, int64_t items, hipStream_t stream) {
  using C = fa::Dkdv64Cfg;
  const int64_t blocks = (int64_t)((ma.max_seqlen_kv + C::BN - 1) / C::BN) * ma.Hk * ma.batch;
  const dim3 grid((unsigned)(ma.sched ? items : blocks)), block(C::NT);
  if (ma.window > 0)  // the window implies the causal bound
    ma.ds ? fa::fa_bwd_dkdv64<true, true, true><<<grid, block, 0, stream>>>(ma)
          : fa::fa_bwd_dkdv64<true, false, true><<<grid, block, 0, stream>>>(ma);
  else if (ma.ds)
    ma.causal ? fa::fa_bwd_dkdv64<true, true, false><<<grid, block, 0, stream>>>(ma)
              : fa::fa_bwd_dkdv64<false, true, false><<<grid, block, 0, stream>>>(ma);
  else
    ma.causal ? fa::fa_bwd_dkdv64<true, false, false><<<grid, block, 0, stream>>>(ma)
              : fa::fa_bwd_dkdv64<false, false, false><<<grid, block, 0, stream>>>(ma);
}

// the stored-dS form's dQ pass over the 64-key kernel's dS blocks: on the dense grid one eight-wave
// workgroup per (256-row q tile, head, sequence); under a host schedule, whose work items are the dQ
// kernel's 128-row q tiles, four-wave workgroups (each wave computes the same sums in either)
template <int NW>
void launch_dq_ds_waves(const fa::MainArgs& ma, int64_t items, hipStream_t stream) {
  using C = fa::DqDsCfg<128, NW>;
  const int64_t blocks = (int64_t)((ma.max_seqlen_q + C::BQ - 1) / C::BQ) * ma.H * ma.batch;
  const dim3 grid((unsigned)(ma.sched ? items : blocks)), block(C::NT);
  if (ma.window > 0)
    fa::fa_bwd_dq_ds<128, true, false, true, true, NW><<<grid, block, 0, stream>>>(ma);
  else if (ma.causal)
    fa::fa_bwd_dq_ds<128, true, false, true, false, NW><<<grid, block, 0, stream>>>(ma);
  else
    fa::fa_bwd_dq_ds<128, true, false, false, false, NW><<<grid, block, 0, stream>>>(ma);
}
void launch_dq_ds(const fa::MainArgs& ma, int64_t items, hipStream_t stream) {
  if (ma.sched)
    launch_dq_ds_waves<4>(ma, items, stream);
  else
    launch_dq_ds_waves<8>(ma, items, stream);
}

// the stored-dS form's dQ pass over the wide-head kernels' dS pieces, for the Q/K head dim padded as the
// wide-head kernels pad it (128, 192 or 256); built here, with the MFMA accumulators in VGPRs, so that
// two four-wave workgroups fit each CU. At 256, on the dense grid, one eight-wave workgroup per CU
// (measured faster there; at 192 the whole step measured slower)
template <int DQ, int NW>
void launch_dq_dsp_waves(const fa::MainArgs& ma, int64_t items, hipStream_t stream) {
  using C = fa::DqDsCfg<DQ, NW>;
  const int64_t blocks = (int64_t)((ma.max_seqlen_q + C::BQ - 1) / C::BQ) * ma.H * ma.batch;
  const dim3 grid((unsigned)(ma.sched ? items : blocks)), block(C::NT);
  if (ma.d_qk == DQ)
    ma.causal ? fa::fa_bwd_dq_ds<DQ, true, true, true, false, NW><<<grid, block, 0, stream>>>(ma)
              : fa::fa_bwd_dq_ds<DQ, true, true, false, false, NW><<<grid, block, 0, stream>>>(ma);
  else
    ma.causal ? fa::fa_bwd_dq_ds<DQ, false, true, true, false, NW><<<grid, block, 0, stream>>>(ma)
              : fa::fa_bwd_dq_ds<DQ, false, true, false, false, NW><<<grid, block, 0, stream>>>(ma);
}
template <int DQ>
void launch_dq_dsp_dim(const fa::MainArgs& ma, int64_t items, hipStream_t stream) {
  if (DQ == 256 && !ma.sched)
    launch_dq_dsp_waves<DQ, 8>(ma, items, stream);
  else
    launch_dq_dsp_waves<DQ, 4>(ma, items, stream);
}
void launch_dq_dsp(const fa::MainArgs& ma, int64_t items, hipStream_t stream) {
  const int pq = ma.d_qk <= 128 ? 128 : ma.d_qk <= 192 ? 192 : 256;
  if (pq == 128)
    launch_dq_dsp_dim<128>(ma, items, stream);
  else if (pq == 192)
    launch_dq_dsp_dim<192>(ma, items, stream);
  else
    launch_dq_dsp_dim<256>(ma, items, stream);
}

// The default takes the stored-dS form where its runs take the 64-key layout, or run the wide-head
// kernels without a window, and the dS workspace stays within this size (on a GPU with 288 GB of
// memory); above it, it keeps the recompute form.
constexpr int64_t kDsDefaultMaxBytes = int64_t(8) << 30;


// The kernels for the padded head dims: each dim rounded up to 64, 128, 192 or 256, and a dim of 64
// next to one above 128 taken as 128.
int padded_dim(int d) { return d <= 64 ? 64 : d <= 128 ? 128 : d <= 192 ? 192 : 256; }

// A window of max_seqlen_q or more hides no key a causal bound would show (query i < max_seqlen_q sees
// every key j <= i either way); the kernels and the schedule take it clamped to max_seqlen_q.
int32_t effective_window(const fa_bwd_desc& d) { return d.window > d.max_seqlen_q ? d.max_seqlen_q : d.window; }

fa::KernelSet pick_kernels(int d_qk, int d_v) {
  int pq = padded_dim(d_qk), pv = padded_dim(d_v);
  if (pq > 128 || pv > 128) {
    if (pq == 64) pq = 128;
    if (pv == 64) pv = 128;
  }
  const bool exact = d_qk == pq && d_v == pv && pq == pv;  // instantiated for equal padded dims
  if (pq == 192 || pv == 192) return fa::wide192_kernel_set(pq, pv, exact);
  if (pq == 256 || pv == 256) return fa::wide_kernel_set(pq, pv, exact);
  if (pq == 64 && pv == 64) return exact ? fa::kernel_set<64, 64, true>() : fa::kernel_set<64, 64, false>();
  if (pq == 128 && pv == 128) return exact ? fa::kernel_set<128, 128, true>() : fa::kernel_set<128, 128, false>();
  return pq == 64 ? fa::kernel_set<64, 128, false>() : fa::kernel_set<128, 64, false>();
}

// Records the next run's four events when profiling is on; nullptr otherwise (or past the limit).
fa_bwd_status next_events(fa_bwd_handle* h, hipEvent_t** out) {
  *out = nullptr;
  if (!h->profiling || h->recorded >= kMaxProfiledRuns) return FA_BWD_OK;
  const size_t base = (size_t)h->recorded * 4;
  if (h->events.size() < base + 4) {
    for (int i = 0; i < 4; ++i) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return FA_BWD_ERR_HIP;
      h->events.push_back(e);
    }
  }
  *out = &h->events[base];
  ++h->recorded;
  return FA_BWD_OK;
}

// The row kernels, one instance per power-of-two threads per row.
template <int TPR>
struct pre_kernel {
  static constexpr auto fn = fa::fa_bwd_pre<TPR, false>;
};
template <int TPR>
struct pre_kernel_exact {  // d_qk = d_v = 8 TPR
  static constexpr auto fn = fa::fa_bwd_pre<TPR, true>;
};
template <int TPR>
struct fill_kernel {
  static constexpr auto fn = fa::fa_fwd_fill<TPR>;
};

template <class Args, template <int> class K>
void launch_rows(int tpr, dim3 grid, hipStream_t stream, const Args& a) {
  switch (tpr) {
    case 1: hipLaunchKernelGGL(K<1>::fn, grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(K<2>::fn, grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(K<4>::fn, grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL(K<8>::fn, grid, dim3(256), 0, stream, a); break;
    case 16: hipLaunchKernelGGL(K<16>::fn, grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(K<32>::fn, grid, dim3(256), 0, stream, a); break;
  }
}

// single-pass main kernel: one workgroup per (kv tile, head, sequence), or per (split, head, sequence)
template <int D, bool SPLIT>
void launch_single_pass(const fa::MainArgs& ma, bool causal, hipStream_t stream) {
  const int64_t first = SPLIT ? fa::kSplits : (ma.max_seqlen_kv + fa::MainCfg<D>::BN - 1) / fa::MainCfg<D>::BN;
  const dim3 grid((unsigned)(first * ma.H * ma.batch));
  if (causal)
    fa::fa_bwd_main<D, true, SPLIT><<<grid, dim3(256), 0, stream>>>(ma);
  else
    fa::fa_bwd_main<D, false, SPLIT><<<grid, dim3(256), 0, stream>>>(ma);
}

template <int D>
void launch_split_reduce(const fa::MainArgs& ma, hipStream_t stream) {
  const dim3 grid((unsigned)((ma.max_seqlen_q + 63) / 64 * ma.H * ma.batch));
  hipLaunchKernelGGL(fa::fa_bwd_split_reduce<D>, grid, dim3(256), 0, stream, ma);
}

template <int D>
void launch_cast(const fa::MainArgs& ma, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = ma.total_q * ma.H;
  hipLaunchKernelGGL(fa::fa_bwd_dq_cast<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                     (const float*)ma.dq_acc, ma.dq, ma.total_q, ma.H, ma.scale);
}

fa_bwd_status launch(fa_bwd_handle* h, const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* m, const float* l, const int32_t* cu_q, const int32_t* cu_kv, float scale,
                     int32_t mask, void* dq, void* dk, void* dv, hipStream_t stream) {
  const fa_bwd_desc& d = h->desc;
  const int padded = (mask == FA_BWD_MASK_PADDING || mask == FA_BWD_MASK_PADDING_CAUSAL) ? 1 : 0;
  const int causal = (mask == FA_BWD_MASK_CAUSAL || mask == FA_BWD_MASK_PADDING_CAUSAL) ? 1 : 0;
  using fa::bf16;

  fa::PreArgs pa;
  pa.o = static_cast<const bf16*>(o);
  pa.dout = static_cast<const bf16*>(dout);
  pa.m = m;
  pa.l = l;
  pa.cu_q = cu_q;
  pa.cu_kv = cu_kv;
  pa.lse2 = h->lse2;
  pa.dvec = h->dvec;
  const bool atomics = h->single_pass && !h->split;
  pa.dq_acc = atomics ? h->dq_acc : nullptr;           // zeroed for the atomics
  pa.dq = atomics ? nullptr : static_cast<bf16*>(dq);  // rows outside every sequence zeroed
  pa.dk = static_cast<bf16*>(dk);
  pa.dv = static_cast<bf16*>(dv);
  pa.total_q = d.total_q;
  pa.total_kv = d.total_kv;
  pa.H = d.num_heads;
  pa.Hk = d.num_heads_kv;
  pa.batch = d.batch;
  pa.max_seqlen_q = d.max_seqlen_q;
  pa.max_seqlen_kv = d.max_seqlen_kv;
  pa.padded = padded;
  pa.d_qk = d.head_dim;
  pa.d_v = d.head_dim_v;
  const int tpr = threads_per_row(d.head_dim, d.head_dim_v);
  const int64_t tokens = d.total_q > d.total_kv ? d.total_q : d.total_kv;
  const int rpb = 256 / tpr;
  hipEvent_t* ev = nullptr;
  const fa_bwd_status es = next_events(h, &ev);
  if (es != FA_BWD_OK) return es;
  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return FA_BWD_ERR_HIP;
  const dim3 pre_grid((unsigned)((tokens + rpb - 1) / rpb * d.num_heads));  // (token group, head) per block
  if (d.head_dim == d.head_dim_v && d.head_dim == 8 * tpr)
    launch_rows<fa::PreArgs, pre_kernel_exact>(tpr, pre_grid, stream, pa);
  else
    launch_rows<fa::PreArgs, pre_kernel>(tpr, pre_grid, stream, pa);
  if (hipGetLastError() != hipSuccess) return FA_BWD_ERR_HIP;
  if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return FA_BWD_ERR_HIP;

  fa::MainArgs ma;
  ma.q = static_cast<const bf16*>(q);
  ma.k = static_cast<const bf16*>(k);
  ma.v = static_cast<const bf16*>(v);
  ma.dout = static_cast<const bf16*>(dout);
  ma.lse2 = h->lse2;
  ma.dvec = h->dvec;
  ma.cu_q = cu_q;
  ma.cu_kv = cu_kv;
  ma.dq_acc = h->dq_acc;
  // the stored-dS form on this run (the 64-key layout's blocks, or the wide-head kernel's pieces)
  const int32_t ds_fmt = h->ds_form ? h->ds_fmt[causal] : kDsNone;
  const bool ds_run = ds_fmt != kDsNone;
  // pieces come from the wide-head kernels only, without a window
  if (ds_fmt == kDsPieces && !ds_pieces_apply(d)) return FA_BWD_ERR_UNSUPPORTED;
  ma.ds = ds_run ? h->ds : nullptr;
  ma.ds_nqs = h->ds_nqs;
  ma.ds_nkt = ds_fmt == kDsPieces ? h->ds_nkt_pieces : h->ds_nkt_blocks;
  ma.dq = static_cast<bf16*>(dq);
  ma.dk = static_cast<bf16*>(dk);
  ma.dv = static_cast<bf16*>(dv);
  ma.total_q = d.total_q;
  ma.total_kv = d.total_kv;
  ma.H = d.num_heads;
  ma.Hk = d.num_heads_kv;
  ma.batch = d.batch;
  ma.max_seqlen_q = d.max_seqlen_q;
  ma.max_seqlen_kv = d.max_seqlen_kv;
  ma.padded = padded;
  ma.causal = causal;
  ma.window = effective_window(d);
  ma.d_qk = d.head_dim;
  ma.d_v = d.head_dim_v;
  ma.scale_log2 = scale * fa::kLog2e;
  ma.scale = scale;
  ma.head_major = 0;
  const fa::KernelSet ks = pick_kernels(d.head_dim, d.head_dim_v);
  const bool planned = h->sched && h->plan_mask == mask;
  ma.sched = planned ? h->sched : nullptr;
  if (h->single_pass) {  // head_dim == head_dim_v, 64 or 128 (checked at create)
    if (d.head_dim == 128)
      h->split ? launch_single_pass<128, true>(ma, causal, stream) : launch_single_pass<128, false>(ma, causal, stream);
    else
      h->split ? launch_single_pass<64, true>(ma, causal, stream) : launch_single_pass<64, false>(ma, causal, stream);
  } else if (!planned || h->n_kv_items > 0) {
    ma.head_major = h->dkdv_head_major[causal] ? 1 : 0;
    if (h->layout[causal] == 3 && !keys64_applies(d)) return FA_BWD_ERR_UNSUPPORTED;  // d = d_v = 128 only
    if (h->layout[causal] == 3)
      launch_dkdv64(ma, h->n_kv_items, stream);
    else
      ks.dkdv(ma, h->n_kv_items, h->layout[causal] == 2, stream);
  }
  if (hipGetLastError() != hipSuccess) return FA_BWD_ERR_HIP;
  if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return FA_BWD_ERR_HIP;

  if (h->single_pass) {
    if (h->split)
      d.head_dim == 128 ? launch_split_reduce<128>(ma, stream) : launch_split_reduce<64>(ma, stream);
    else
      d.head_dim == 128 ? launch_cast<128>(ma, stream) : launch_cast<64>(ma, stream);
  } else if (!planned || h->n_q_items > 0) {
    ma.sched = planned ? h->sched + 2 * h->n_kv_items : nullptr;
    ma.head_major = (ds_run ? h->ds_head_major[causal] : h->dq_head_major[causal]) ? 1 : 0;
    if (ds_fmt == kDsPieces)
      launch_dq_dsp(ma, h->n_q_items, stream);
    else if (ds_run)
      launch_dq_ds(ma, h->n_q_items, stream);
    else
      ks.dq(ma, h->n_q_items, h->dq_split, stream);
  }
  if (hipGetLastError() != hipSuccess) return FA_BWD_ERR_HIP;
  if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return FA_BWD_ERR_HIP;
  return FA_BWD_OK;
}

fa_bwd_status launch_fwd(fa_bwd_handle* h, const void* q, const void* k, const void* v, const int32_t* cu_q,
                         const int32_t* cu_kv, float scale, int32_t mask, void* o, float* m, float* l,
                         hipStream_t stream) {
  const fa_bwd_desc& d = h->desc;
  const int padded = (mask == FA_BWD_MASK_PADDING || mask == FA_BWD_MASK_PADDING_CAUSAL) ? 1 : 0;
  const bool causal = mask == FA_BWD_MASK_CAUSAL || mask == FA_BWD_MASK_PADDING_CAUSAL;
  using fa::bf16;
  fa::FwdArgs fa;
  fa.q = static_cast<const bf16*>(q);
  fa.k = static_cast<const bf16*>(k);
  fa.v = static_cast<const bf16*>(v);
  fa.cu_q = cu_q;
  fa.cu_kv = cu_kv;
  fa.o = static_cast<bf16*>(o);
  fa.m = m;
  fa.l = l;
  fa.total_q = d.total_q;
  fa.total_kv = d.total_kv;
  fa.H = d.num_heads;
  fa.Hk = d.num_heads_kv;
  fa.batch = d.batch;
  fa.max_seqlen_q = d.max_seqlen_q;
  fa.max_seqlen_kv = d.max_seqlen_kv;
  fa.padded = padded;
  fa.window = effective_window(d);
  fa.d_qk = d.head_dim;
  fa.d_v = d.head_dim_v;
  fa.scale_log2 = scale * fa::kLog2e;
  hipEvent_t* ev = nullptr;
  const fa_bwd_status es = next_events(h, &ev);
  if (es != FA_BWD_OK) return es;
  const int tpr = threads_per_row(d.head_dim_v, d.head_dim_v);
  const int rpb = 256 / tpr;
  const int64_t rows = d.total_q * d.num_heads;
  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return FA_BWD_ERR_HIP;
  launch_rows<fa::FwdArgs, fill_kernel>(tpr, dim3((unsigned)((rows + rpb - 1) / rpb)), stream, fa);
  if (hipGetLastError() != hipSuccess) return FA_BWD_ERR_HIP;
  if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return FA_BWD_ERR_HIP;
  const bool planned = h->sched && h->plan_mask == mask;
  fa.sched = planned ? h->sched + 2 * h->n_kv_items : nullptr;
  if (!planned || h->n_q_items > 0) pick_kernels(d.head_dim, d.head_dim_v).fwd(fa, causal, h->n_q_items, stream);
  if (hipGetLastError() != hipSuccess) return FA_BWD_ERR_HIP;
  if (ev && (hipEventRecord(ev[2], stream) != hipSuccess || hipEventRecord(ev[3], stream) != hipSuccess))
    return FA_BWD_ERR_HIP;
  return FA_BWD_OK;
}

void drop_plan(fa_bwd_handle* h) {
  if (h->sched) (void)hipFree(h->sched);
  h->sched = nullptr;
  h->n_kv_items = h->n_q_items = 0;
}

// The work items of the recompute kernels for host sequence offsets, longest first. Work counts the
// tile pairs a workgroup visits, as the kernels bound their loops (causal start, window band).
fa_bwd_status build_plan(const fa_bwd_desc& d, int32_t layout, const int32_t* cq, const int32_t* ck, int32_t mask,
                         std::vector<int32_t>& out, int64_t& n_kv, int64_t& n_q) {
  const bool padded = mask == FA_BWD_MASK_PADDING || mask == FA_BWD_MASK_PADDING_CAUSAL;
  const bool causal = mask == FA_BWD_MASK_CAUSAL || mask == FA_BWD_MASK_PADDING_CAUSAL || d.window > 0;
  if (cq[0] != 0 || ck[0] != 0) return FA_BWD_ERR_INVALID_ARGUMENT;
  for (int b = 0; b < d.batch; ++b) {
    const int64_t lq = (int64_t)cq[b + 1] - cq[b], lk = (int64_t)ck[b + 1] - ck[b];
    if (lq < 0 || lk < 0 || lq > d.max_seqlen_q || lk > d.max_seqlen_kv) return FA_BWD_ERR_INVALID_ARGUMENT;
  }
  if (padded ? ((int64_t)d.batch * d.max_seqlen_q > d.total_q || (int64_t)d.batch * d.max_seqlen_kv > d.total_kv)
             : (cq[d.batch] > d.total_q || ck[d.batch] > d.total_kv))
    return FA_BWD_ERR_INVALID_ARGUMENT;
  const fa::KernelSet ks = pick_kernels(d.head_dim, d.head_dim_v);
  // kv rows per dK/dV workgroup and q rows per step of the layout the runs take
  const int kv_tile = layout == 3 ? fa::Dkdv64Cfg::BN : ks.kv_tile;
  const int q_step = layout == 3 ? fa::Dkdv64Cfg::BM : ks.q_step;
  struct Item {
    int64_t work;
    int32_t tile, hb;
  };
  std::vector<Item> kv, q;
  const int G = d.num_heads / d.num_heads_kv, w = effective_window(d);
  for (int b = 0; b < d.batch; ++b) {
    const int lq = cq[b + 1] - cq[b], lk = ck[b + 1] - ck[b];
    const int n_qs = (lq + q_step - 1) / q_step;  // q steps of the dK/dV kernel
    for (int t = 0; t * kv_tile < lk; ++t) {
      const int kv0 = t * kv_tile;
      const int qt0 = causal ? kv0 / q_step : 0;
      const int qt_end = w > 0 ? std::min(n_qs, (kv0 + kv_tile - 2 + w) / q_step + 1) : n_qs;
      const int64_t work = (int64_t)G * std::max(0, qt_end - qt0);
      for (int hk = 0; hk < d.num_heads_kv; ++hk) kv.push_back({work, t, b * d.num_heads_kv + hk});
    }
    for (int t = 0; t * ks.q_tile < lq; ++t) {
      const int i0 = t * ks.q_tile;
      int n_kt = (lk + ks.kv_step - 1) / ks.kv_step;
      if (causal) n_kt = std::min(n_kt, (i0 + ks.q_tile - 1) / ks.kv_step + 1);
      const int t0 = w > 0 ? std::max(0, i0 - w + 1) / ks.kv_step : 0;
      const int64_t work = std::max(0, n_kt - t0);
      for (int hq = 0; hq < d.num_heads; ++hq) q.push_back({work, t, b * d.num_heads + hq});
    }
  }
  // most work first; ties in the dense grid's order (tile, then sequence and head)
  auto longest_first = [](const Item& x, const Item& y) {
    if (x.work != y.work) return x.work > y.work;
    return x.tile != y.tile ? x.tile < y.tile : x.hb < y.hb;
  };
  std::sort(kv.begin(), kv.end(), longest_first);
  std::sort(q.begin(), q.end(), longest_first);
  out.clear();
  for (const Item& it : kv) out.insert(out.end(), {it.tile, it.hb});
  for (const Item& it : q) out.insert(out.end(), {it.tile, it.hb});
  n_kv = (int64_t)kv.size();
  n_q = (int64_t)q.size();
  return FA_BWD_OK;
}

// The dK/dV layout an algorithm code forces (0: chosen by the rule).
int32_t dkdv_layout_code(int32_t algorithm) {
  switch (algorithm) {
    case FA_BWD_ALGO_RECOMPUTE_DQ_8W: return 1;
    case FA_BWD_ALGO_RECOMPUTE_DQ_4W: return 2;
    case FA_BWD_ALGO_RECOMPUTE_DQ_64K:
    case FA_BWD_ALGO_STORED_DS: return 3;
    default: return 0;
  }
}

// The kv-outer kernel's layout and the dense grids' orders for runs without and with a causal bound,
// from the descriptor (every sequence taken at the maximum lengths) and the compute-unit count.
void configure_layouts(fa_bwd_handle* h, int cus) {
  const fa_bwd_desc& hd = h->desc;
  h->dq_split = dq_key_split(hd, pick_kernels(hd.head_dim, hd.head_dim_v).two_layouts, cus);
  const int64_t per_tile_heads = (int64_t)hd.batch * hd.num_heads;  // Hk K/V heads x G query heads each
  const int G = hd.num_heads / hd.num_heads_kv;
  for (int c = 0; c < 2; ++c) {
    int64_t total = 0, largest = 0;
    dkdv_work(hd.max_seqlen_q, hd.max_seqlen_kv, c == 1 || hd.window > 0, effective_window(hd), total, largest);
    h->four_dense[c] = four_waves_balances((double)total * (double)per_tile_heads, (double)largest * G, cus);
    // heads up to 128: two workgroups per CU in the dQ kernel and the four-wave dK/dV layout, one in
    // the eight-wave one and the 64-key one; wider heads: one in both kernels
    const int64_t kv_heads_x_seqs = (int64_t)hd.batch * hd.num_heads_kv;
    const bool narrow = pick_kernels(hd.head_dim, hd.head_dim_v).two_layouts;
    const bool four = narrow && (h->dkdv_layout == 2 || (h->dkdv_layout == 0 && h->four_dense[c]));
    // the 64-key layout's own tile sizes: 256 keys, 32-row q steps
    int64_t total64 = 0, largest64 = 0;
    if (keys64_applies(hd))
      dkdv_work(hd.max_seqlen_q, hd.max_seqlen_kv, c == 1 || hd.window > 0, effective_window(hd), total64,
                largest64, fa::Dkdv64Cfg::BN, fa::Dkdv64Cfg::BM);
    // (forced by FA_BWD_ALGO_RECOMPUTE_DQ_64K, or by FA_BWD_ALGO_STORED_DS at head dims of 128: with a head
    // dim above 128 the stored-dS form runs on the wide-head kernels)
    const bool keys64 = keys64_applies(hd) && (h->dkdv_layout == 3 ||
                        (h->dkdv_layout == 0 && hd.window == 0 &&
                         keys64_balances((double)total64 * (double)per_tile_heads, (double)largest64 * G, cus)));
    h->layout[c] = keys64 ? 3 : four ? 2 : 1;
    if (keys64) {
      total = total64;
      largest = largest64;
    }
    h->dkdv_head_major[c] = head_major_balances((double)total * (double)per_tile_heads, (double)largest * G,
                                                (int64_t)cus * (four && h->layout[c] == 2 ? 2 : 1),
                                                kv_heads_x_seqs);
    int64_t qtotal = 0, qlargest = 0;
    dq_work(hd.max_seqlen_q, hd.max_seqlen_kv, c == 1 || hd.window > 0, effective_window(hd), qtotal, qlargest);
    h->dq_head_major[c] = head_major_balances((double)qtotal * (double)per_tile_heads, (double)qlargest,
                                              (int64_t)cus * (narrow && !h->dq_split ? 2 : 1), per_tile_heads);
    // the stored-dS pass: counted as 128-row tiles, two per CU; its eight-wave workgroups (256 rows, one
    // per CU) double the largest item and halve the slots, the same product
    h->ds_head_major[c] = head_major_balances((double)qtotal * (double)per_tile_heads, (double)qlargest,
                                              (int64_t)cus * 2, per_tile_heads);
  }
}

// Host checks shared by fa_bwd_run and fa_fwd_run.
fa_bwd_status check_run(const fa_bwd_handle* h, float scale, int32_t mask) {
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_BWD_ERR_INVALID_ARGUMENT;
  if (mask < FA_BWD_MASK_NONE || mask > FA_BWD_MASK_PADDING_CAUSAL) return FA_BWD_ERR_INVALID_ARGUMENT;
  const fa_bwd_desc& d = h->desc;
  if (mask == FA_BWD_MASK_PADDING || mask == FA_BWD_MASK_PADDING_CAUSAL) {
    if ((int64_t)d.batch * d.max_seqlen_q > d.total_q || (int64_t)d.batch * d.max_seqlen_kv > d.total_kv)
      return FA_BWD_ERR_INVALID_ARGUMENT;
  }
  return FA_BWD_OK;
}

// (m, l) or, with l null, the log-sum-exp in m: shared checks and launch of both backward entries.
fa_bwd_status check_pointers(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* m, const float* l, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_kv, void* dq, void* dk, void* dv) {
  if (!q || !k || !v || !o || !dout || !m || !cu_seqlens_q || !cu_seqlens_kv || !dq || !dk || !dv)
    return FA_BWD_ERR_INVALID_ARGUMENT;
  const void* vec[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : vec)
    if (!aligned(p, 16)) return FA_BWD_ERR_INVALID_ARGUMENT;
  if (!aligned(m, 4) || (l && !aligned(l, 4)) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_kv, 4))
    return FA_BWD_ERR_INVALID_ARGUMENT;
  return FA_BWD_OK;
}

fa_bwd_status run_common(fa_bwd_handle* h, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* m, const float* l, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_kv, float scale, int32_t mask, void* dq, void* dk, void* dv,
                         void* stream) {
  if (!h) return FA_BWD_ERR_INVALID_ARGUMENT;
  const fa_bwd_status ps = check_pointers(q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, dq, dk, dv);
  if (ps != FA_BWD_OK) return ps;
  const fa_bwd_status cs = check_run(h, scale, mask);
  if (cs != FA_BWD_OK) return cs;
  return launch(h, q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, scale, mask, dq, dk, dv,
                static_cast<hipStream_t>(stream));
}

// ---- the allocation-free entry point's scratch: the two fp32 [H][total_q] row-statistic arrays
// (lse2, then D) of one run, for total_q x num_heads up to kNoAllocMaxRows, in a file-scope device array
// that each GPU holds from the time the library's code is loaded on it until the process ends. Host code
// never uses the array's name as an address: the device address comes from hipGetSymbolAddress, once
// per device, with that device current.
constexpr int64_t kNoAllocMaxRows = int64_t(1) << 22;  // 2 x 4 x 2^22 bytes = 32 MiB
constexpr int kNoAllocMaxDevices = 64;

struct NoAllocDevice {
  float* scratch;  // device address of `scratch` on this device
  int cus;         // its compute units (for the layout rule)
};

std::mutex g_noalloc_mutex;
NoAllocDevice g_noalloc[kNoAllocMaxDevices];
bool g_noalloc_ready[kNoAllocMaxDevices];

}  // namespace

static __device__ __align__(256) float scratch[2 * kNoAllocMaxRows];

namespace {

// The scratch address and compute-unit count of the current device, looked up on its first use.
fa_bwd_status noalloc_device(NoAllocDevice* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_BWD_ERR_HIP;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return FA_BWD_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_noalloc_mutex);
  if (!g_noalloc_ready[dev]) {
    void* ptr = nullptr;
    int cus = 0;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_BWD_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return FA_BWD_ERR_HIP;
    g_noalloc[dev] = {static_cast<float*>(ptr), cus};
    g_noalloc_ready[dev] = true;
  }
  *out = g_noalloc[dev];
  return FA_BWD_OK;
}

}  // namespace

extern "C" {

fa_bwd_status fa_bwd_create(const fa_bwd_desc* desc, fa_bwd_handle** out) {
  if (!out) return FA_BWD_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  const fa_bwd_status st = check_desc(desc);
  if (st != FA_BWD_OK) return st;
  fa_bwd_handle* h = new (std::nothrow) fa_bwd_handle();
  if (!h) return FA_BWD_ERR_OUT_OF_MEMORY;
  h->desc = *desc;
  if (h->desc.num_heads_kv == 0) h->desc.num_heads_kv = desc->num_heads;
  if (h->desc.head_dim_v == 0) h->desc.head_dim_v = desc->head_dim;
  h->single_pass = desc->algorithm == FA_BWD_ALGO_SINGLE_PASS || desc->algorithm == FA_BWD_ALGO_SPLIT_REDUCE;
  h->split = desc->algorithm == FA_BWD_ALGO_SPLIT_REDUCE;
  h->dkdv_layout = dkdv_layout_code(desc->algorithm);
  int cus = 0;
  if (hipGetDevice(&h->device) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess || cus < 1) {
    delete h;
    return FA_BWD_ERR_HIP;
  }
  configure_layouts(h, cus);
  // the dS format of runs without and with a causal bound: the explicit form everywhere its kernels run,
  // the default where it is faster (the 64-key layout, wide heads without a window) and its workspace
  // stays within kDsDefaultMaxBytes. (The 128-key layouts could store pieces too, but their stores cost
  // more than the dQ pass saves.)
  const int64_t need_blocks = ds_bytes_of(h->desc, false, h->ds_nqs, h->ds_nkt_blocks);
  const int64_t need_pieces = ds_bytes_of(h->desc, true, h->ds_nqs, h->ds_nkt_pieces);
  const bool d128 = h->desc.head_dim == 128 && h->desc.head_dim_v == 128;
  const bool explicit_ds = desc->algorithm == FA_BWD_ALGO_STORED_DS;
  int64_t ds_need = 0;
  h->ds_form = false;
  for (int c = 0; c < 2; ++c) {
    int32_t fmt = kDsNone;
    if (ds_pieces_apply(h->desc))
      fmt = kDsPieces;
    else if (d128 && h->layout[c] == 3)
      fmt = kDsBlocks;
    const int64_t need = fmt == kDsBlocks ? need_blocks : fmt == kDsPieces ? need_pieces : 0;
    if (!explicit_ds && (desc->algorithm != FA_BWD_ALGO_DEFAULT || need < 0 || need > kDsDefaultMaxBytes))
      fmt = kDsNone;
    h->ds_fmt[c] = fmt;
    if (fmt != kDsNone) {
      h->ds_form = true;
      ds_need = std::max(ds_need, need);
    }
  }
  const size_t ds_bytes = h->ds_form ? (size_t)ds_need : 0;
  const size_t stats = (size_t)desc->total_q * desc->num_heads;
  const size_t acc = stats * desc->head_dim * (h->split ? fa::kSplits : 1);
  if ((h->single_pass && hipMalloc(&h->dq_acc, acc * sizeof(float)) != hipSuccess) ||
      (h->ds_form && hipMalloc(&h->ds, ds_bytes) != hipSuccess) ||
      hipMalloc(&h->lse2, stats * sizeof(float)) != hipSuccess ||
      hipMalloc(&h->dvec, stats * sizeof(float)) != hipSuccess) {
    (void)hipGetLastError();
    if (h->dq_acc) (void)hipFree(h->dq_acc);
    if (h->ds) (void)hipFree(h->ds);
    if (h->lse2) (void)hipFree(h->lse2);
    if (h->dvec) (void)hipFree(h->dvec);
    delete h;
    return FA_BWD_ERR_OUT_OF_MEMORY;
  }
  *out = h;
  return FA_BWD_OK;
}

fa_bwd_status fa_bwd_run(fa_bwd_handle* h, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* m, const float* l, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_kv, float scale, int32_t mask, void* dq, void* dk, void* dv,
                         void* stream) {
  if (!l) return FA_BWD_ERR_INVALID_ARGUMENT;
  return run_common(h, q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, scale, mask, dq, dk, dv, stream);
}

fa_bwd_status fa_bwd_run_lse(fa_bwd_handle* h, const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_kv, float scale, int32_t mask, void* dq, void* dk, void* dv,
                             void* stream) {
  if (!lse) return FA_BWD_ERR_INVALID_ARGUMENT;
  return run_common(h, q, k, v, o, dout, lse, nullptr, cu_seqlens_q, cu_seqlens_kv, scale, mask, dq, dk, dv, stream);
}

fa_bwd_status fa_bwd_run_noalloc(const fa_bwd_desc* desc, const void* q, const void* k, const void* v,
                                 const void* o, const void* dout, const float* m, const float* l,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, float scale,
                                 int32_t mask, void* dq, void* dk, void* dv, void* stream) {
  const fa_bwd_status ds = check_desc(desc);
  if (ds != FA_BWD_OK) return ds;
  if (desc->algorithm == FA_BWD_ALGO_SINGLE_PASS || desc->algorithm == FA_BWD_ALGO_SPLIT_REDUCE ||
      desc->algorithm == FA_BWD_ALGO_STORED_DS)
    return FA_BWD_ERR_UNSUPPORTED;  // their dQ (or dS) workspace is not part of the fixed scratch
  if (desc->total_q > kNoAllocMaxRows / desc->num_heads) return FA_BWD_ERR_SCRATCH_LIMIT;
  if (!l) return FA_BWD_ERR_INVALID_ARGUMENT;
  const fa_bwd_status ps = check_pointers(q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, dq, dk, dv);
  if (ps != FA_BWD_OK) return ps;
  // a handle on the stack (its event list stays empty, so nothing is allocated) that points at the scratch
  fa_bwd_handle h{};
  h.desc = *desc;
  if (h.desc.num_heads_kv == 0) h.desc.num_heads_kv = desc->num_heads;
  if (h.desc.head_dim_v == 0) h.desc.head_dim_v = desc->head_dim;
  h.dkdv_layout = dkdv_layout_code(desc->algorithm);
  const fa_bwd_status cs = check_run(&h, scale, mask);
  if (cs != FA_BWD_OK) return cs;
  NoAllocDevice nd;
  const fa_bwd_status ns = noalloc_device(&nd);
  if (ns != FA_BWD_OK) return ns;
  (void)hipGetDevice(&h.device);
  configure_layouts(&h, nd.cus);
  h.lse2 = nd.scratch;
  h.dvec = nd.scratch + desc->total_q * desc->num_heads;
  return launch(&h, q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, scale, mask, dq, dk, dv,
                static_cast<hipStream_t>(stream));
}

fa_bwd_status fa_fwd_run(fa_bwd_handle* h, const void* q, const void* k, const void* v,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, float scale, int32_t mask,
                         void* o, float* m, float* l, void* stream) {
  if (!h || !q || !k || !v || !cu_seqlens_q || !cu_seqlens_kv || !o || !m || !l) return FA_BWD_ERR_INVALID_ARGUMENT;
  const void* vec[] = {q, k, v, o};
  for (const void* p : vec)
    if (!aligned(p, 16)) return FA_BWD_ERR_INVALID_ARGUMENT;
  if (!aligned(m, 4) || !aligned(l, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_kv, 4))
    return FA_BWD_ERR_INVALID_ARGUMENT;
  const fa_bwd_status cs = check_run(h, scale, mask);
  if (cs != FA_BWD_OK) return cs;
  return launch_fwd(h, q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, mask, o, m, l, static_cast<hipStream_t>(stream));
}

fa_bwd_status fa_bwd_plan(fa_bwd_handle* h, const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_kv_host,
                          int32_t mask) {
  if (!h) return FA_BWD_ERR_INVALID_ARGUMENT;
  if (h->single_pass) return FA_BWD_ERR_UNSUPPORTED;
  if (!cu_seqlens_q_host != !cu_seqlens_kv_host) return FA_BWD_ERR_INVALID_ARGUMENT;
  if (cu_seqlens_q_host && (mask < FA_BWD_MASK_NONE || mask > FA_BWD_MASK_PADDING_CAUSAL))
    return FA_BWD_ERR_INVALID_ARGUMENT;
  std::vector<int32_t> items;
  int64_t n_kv = 0, n_q = 0;
  if (cu_seqlens_q_host) {
    const bool causal = mask == FA_BWD_MASK_CAUSAL || mask == FA_BWD_MASK_PADDING_CAUSAL;
    const fa_bwd_status st =
        build_plan(h->desc, h->layout[causal ? 1 : 0], cu_seqlens_q_host, cu_seqlens_kv_host, mask, items, n_kv, n_q);
    if (st != FA_BWD_OK) return st;
  }
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(h->device) != hipSuccess) return FA_BWD_ERR_HIP;
  fa_bwd_status st = FA_BWD_OK;
  if (h->sched && hipDeviceSynchronize() != hipSuccess) st = FA_BWD_ERR_HIP;  // runs may still read it
  drop_plan(h);
  if (st == FA_BWD_OK && !items.empty()) {
    if (hipMalloc(&h->sched, items.size() * sizeof(int32_t)) != hipSuccess) {
      (void)hipGetLastError();
      h->sched = nullptr;
      st = FA_BWD_ERR_OUT_OF_MEMORY;
    } else if (hipMemcpy(h->sched, items.data(), items.size() * sizeof(int32_t), hipMemcpyHostToDevice) !=
               hipSuccess) {
      drop_plan(h);
      st = FA_BWD_ERR_HIP;
    } else {
      h->n_kv_items = n_kv;
      h->n_q_items = n_q;
      h->plan_mask = mask;
    }
  }
  (void)hipSetDevice(prev);
  return st;
}

fa_bwd_status fa_bwd_destroy(fa_bwd_handle* h) {
  if (!h) return FA_BWD_OK;
  int prev = 0;
  fa_bwd_status st = FA_BWD_OK;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(h->device) != hipSuccess) st = FA_BWD_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) st = FA_BWD_ERR_HIP;
  if (h->dq_acc && hipFree(h->dq_acc) != hipSuccess) st = FA_BWD_ERR_HIP;
  if (h->ds && hipFree(h->ds) != hipSuccess) st = FA_BWD_ERR_HIP;
  if (hipFree(h->lse2) != hipSuccess) st = FA_BWD_ERR_HIP;
  if (hipFree(h->dvec) != hipSuccess) st = FA_BWD_ERR_HIP;
  drop_plan(h);
  release_events(h);
  (void)hipSetDevice(prev);
  delete h;
  return st;
}

const char* fa_bwd_status_string(fa_bwd_status s) {
  switch (s) {
    case FA_BWD_OK: return "ok";
    case FA_BWD_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FA_BWD_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_BWD_ERR_OUT_OF_MEMORY: return "out of device memory";
    case FA_BWD_ERR_HIP: return "HIP runtime error";
    case FA_BWD_ERR_SCRATCH_LIMIT: return "problem exceeds the fixed scratch of fa_bwd_run_noalloc";
  }
  return "unknown status";
}

const fa_bwd_desc* fa_bwd_get_desc(const fa_bwd_handle* h) { return h ? &h->desc : nullptr; }

int32_t fa_bwd_dkdv_layout(const fa_bwd_handle* h, int32_t mask) {
  if (!h || mask < FA_BWD_MASK_NONE || mask > FA_BWD_MASK_PADDING_CAUSAL) return -1;
  if (h->single_pass) return h->split ? FA_BWD_ALGO_SPLIT_REDUCE : FA_BWD_ALGO_SINGLE_PASS;
  if (!pick_kernels(h->desc.head_dim, h->desc.head_dim_v).two_layouts)  // wide heads: one layout
    return FA_BWD_ALGO_RECOMPUTE_DQ;
  const bool causal = mask == FA_BWD_MASK_CAUSAL || mask == FA_BWD_MASK_PADDING_CAUSAL;
  switch (h->layout[causal]) {
    case 3: return FA_BWD_ALGO_RECOMPUTE_DQ_64K;
    case 2: return FA_BWD_ALGO_RECOMPUTE_DQ_4W;
    default: return FA_BWD_ALGO_RECOMPUTE_DQ_8W;
  }
}

int32_t fa_bwd_dq_form(const fa_bwd_handle* h, int32_t mask) {
  if (!h || mask < FA_BWD_MASK_NONE || mask > FA_BWD_MASK_PADDING_CAUSAL) return -1;
  if (h->single_pass) return h->split ? FA_BWD_ALGO_SPLIT_REDUCE : FA_BWD_ALGO_SINGLE_PASS;
  const bool causal = mask == FA_BWD_MASK_CAUSAL || mask == FA_BWD_MASK_PADDING_CAUSAL;
  return h->ds_form && h->ds_fmt[causal] != kDsNone ? FA_BWD_ALGO_STORED_DS : FA_BWD_ALGO_RECOMPUTE_DQ;
}

fa_bwd_status fa_bwd_profile_enable(fa_bwd_handle* h, int32_t enable) {
  if (!h) return FA_BWD_ERR_INVALID_ARGUMENT;
  fa_bwd_status st = FA_BWD_OK;
  if (!h->events.empty() && hipDeviceSynchronize() != hipSuccess) st = FA_BWD_ERR_HIP;
  release_events(h);
  h->profiling = enable != 0;
  return st;
}

fa_bwd_status fa_bwd_profile_collect(fa_bwd_handle* h, float* ms, int32_t max_runs, int32_t* n_runs) {
  if (!h || !n_runs || max_runs < 0 || (max_runs > 0 && !ms)) return FA_BWD_ERR_INVALID_ARGUMENT;
  *n_runs = 0;
  const int64_t n = h->recorded < max_runs ? h->recorded : max_runs;
  for (int64_t r = 0; r < n; ++r) {
    hipEvent_t* e = &h->events[(size_t)r * 4];
    if (hipEventSynchronize(e[3]) != hipSuccess) return FA_BWD_ERR_HIP;
    for (int s = 0; s < 3; ++s)
      if (hipEventElapsedTime(&ms[r * 3 + s], e[s], e[s + 1]) != hipSuccess) return FA_BWD_ERR_HIP;
  }
  *n_runs = (int32_t)n;
  // keep the events for reuse, forget the runs
  h->recorded = 0;
  return FA_BWD_OK;
}

}  // extern "C"

