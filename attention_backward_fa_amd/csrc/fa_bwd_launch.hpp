// fa_bwd_launch.hpp -- launches of the recompute-form kernels (dK/dV, dQ) and of the forward for one
// pair of padded head dims (DQ for Q and K, DV for V, O and dO). The pairs with a dim above 128 are
// instantiated only in fa_bwd_wide.hip and fa_bwd_wide192.hip, which are compiled with MFMA
// accumulators allowed in the AGPRs: their accumulators need more registers than the 256 VGPRs of
// one wave.
#pragma once
#include "fa_bwd_kernels.hpp"

namespace fa {

// EXACT: the head dims equal the padded ones, so the kernels take them as constants.
template <int DQ, int DV, bool EXACT>
struct Recompute {
  // workgroups of the dK/dV kernel: (kv tile, K/V head, sequence), kv tiles outermost
  static int64_t dkdv_blocks(const MainArgs& a) {
    return (int64_t)((a.max_seqlen_kv + DkdvCfg<DQ, DV>::BN - 1) / DkdvCfg<DQ, DV>::BN) * a.Hk * a.batch;
  }
  // workgroups of the dQ kernel and of the forward: (q tile, head, sequence), q tiles outermost
  static int64_t q_blocks(int max_seqlen_q, int H, int batch) {
    return (int64_t)((max_seqlen_q + DqCfg<DQ, DV>::BQ - 1) / DqCfg<DQ, DV>::BQ) * H * batch;
  }

  template <int NMT>
  static void dkdv_layout(const MainArgs& a, int64_t items, hipStream_t s) {
    const dim3 grid((unsigned)(a.sched ? items : dkdv_blocks(a))), block(DkdvCfg<DQ, DV, NMT>::NT);
    if (a.window > 0)  // the window implies the causal bound
      fa_bwd_dkdv<DQ, DV, true, true, EXACT, NMT><<<grid, block, 0, s>>>(a);
    else if (a.causal)
      fa_bwd_dkdv<DQ, DV, true, false, EXACT, NMT><<<grid, block, 0, s>>>(a);
    else
      fa_bwd_dkdv<DQ, DV, false, false, EXACT, NMT><<<grid, block, 0, s>>>(a);
  }
  // items: the workgroup count of a host schedule (a.sched), else unused; four_waves: the four-wave
  // layout (heads up to 128; wider heads have one layout per pair of head dims: one M-tile per step
  // where both outputs' accumulators fit one wave, same tiles and order of every sum as two M-tiles,
  // without the P/dS swap; else two)
  static void dkdv(const MainArgs& a, int64_t items, bool four_waves, hipStream_t s) {
    if constexpr (DkdvCfg<DQ, DV>::WIDE && DQ + DV <= 320)  // accumulators of both outputs fit one wave
      dkdv_layout<1>(a, items, s);
    else if constexpr (DkdvCfg<DQ, DV>::WIDE)
      dkdv_layout<2>(a, items, s);
    else if (four_waves)
      dkdv_layout<1>(a, items, s);
    else
      dkdv_layout<2>(a, items, s);
  }

  template <int KS>
  static void dq_groups(const MainArgs& a, int64_t items, hipStream_t s) {
    const dim3 grid((unsigned)(a.sched ? items : q_blocks(a.max_seqlen_q, a.H, a.batch))),
        block(DqCfg<DQ, DV>::NT * KS);
    if (a.window > 0)
      fa_bwd_dq<DQ, DV, true, true, EXACT, KS><<<grid, block, 0, s>>>(a);
    else if (a.causal)
      fa_bwd_dq<DQ, DV, true, false, EXACT, KS><<<grid, block, 0, s>>>(a);
    else
      fa_bwd_dq<DQ, DV, false, false, EXACT, KS><<<grid, block, 0, s>>>(a);
  }
  // key_split: two groups of four waves per workgroup, each over every other kv step (heads up to
  // 128; wider heads have one form)
  static void dq(const MainArgs& a, int64_t items, bool key_split, hipStream_t s) {
    if constexpr (!DqCfg<DQ, DV>::WIDE) {
      if (key_split) return dq_groups<2>(a, items, s);
    }
    dq_groups<1>(a, items, s);
  }

  static void fwd(const FwdArgs& a, bool causal, int64_t items, hipStream_t s) {
    const dim3 grid((unsigned)(a.sched ? items : q_blocks(a.max_seqlen_q, a.H, a.batch))), block(DqCfg<DQ, DV>::NT);
    if (a.window > 0)
      fa_fwd<DQ, DV, true, true, EXACT><<<grid, block, 0, s>>>(a);
    else if (causal)
      fa_fwd<DQ, DV, true, false, EXACT><<<grid, block, 0, s>>>(a);
    else
      fa_fwd<DQ, DV, false, false, EXACT><<<grid, block, 0, s>>>(a);
  }
};

// The launches of one pair of padded head dims, and the tile sizes a host schedule counts in.
struct KernelSet {
  void (*dkdv)(const MainArgs&, int64_t, bool, hipStream_t);
  void (*dq)(const MainArgs&, int64_t, bool, hipStream_t);
  void (*fwd)(const FwdArgs&, bool, int64_t, hipStream_t);
  int kv_tile, q_step;  // dK/dV kernel: kv rows per workgroup, q rows per step (eight-wave layout)
  bool two_layouts;     // the dK/dV kernel also has the four-wave layout
  int q_tile, kv_step;  // dQ kernel and forward: q rows per workgroup, kv rows per step
};

template <int DQ, int DV, bool EXACT>
KernelSet kernel_set() {
  using R = Recompute<DQ, DV, EXACT>;
  return {R::dkdv, R::dq, R::fwd, DkdvCfg<DQ, DV>::BN, DkdvCfg<DQ, DV>::BM, !DkdvCfg<DQ, DV>::WIDE,
          DqCfg<DQ, DV>::BQ, DqCfg<DQ, DV>::BK};
}

// The pairs (128, 256), (256, 128) and (256, 256), from fa_bwd_wide.hip; pq, pv are padded dims,
// exact that the head dims equal them (pq = pv = 256).
KernelSet wide_kernel_set(int pq, int pv, bool exact);
// The pairs with a 192 (the other 128, 192 or 256), from fa_bwd_wide192.hip; exact: pq = pv = 192 and
// the head dims equal them.
KernelSet wide192_kernel_set(int pq, int pv, bool exact);

}  // namespace fa
