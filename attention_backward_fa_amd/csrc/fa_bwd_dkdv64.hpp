// fa_bwd_dkdv64.hpp -- dK and dV of the recompute form for head dims of 128 with 64 keys per wave.
//
// Steps 1-3 and 5-7 of the per-tile math of the PyPTO-Gym SK-16 article (section 3.1) for one
// 256-key tile of one (K/V head, sequence): S = Q K^T, P = exp2(S*scale*log2e - lse2),
// dP = dO V^T, dS = P (dP - D), dV += P^T dO, dK += dS^T Q, with dK scaled once at the end.
// WINDOW (with the causal bound): query i sees keys (i - window, i] only (the jax cuDNN wrapper's
// sliding window); the steps end at the last query row that sees a key of the tile.
//
// Layout (one workgroup of four waves per CU, one wave per SIMD):
//   - wave w owns keys kv0 + 64 w .. + 63 as two 32-key MFMA tiles; the first 64 features of its K
//     rows sit in registers as B-operand fragments of S = Q K^T, the other 64 in an LDS tile; its dK,
//     dV sums (2 x 64 x 128 fp32 per wave) sit in the accumulator registers for the whole kernel;
//   - the V tile (256 keys) is loaded into LDS once; Q and dO tiles of 32 query rows stream through
//     three LDS buffers with LDS-DMA, two steps ahead of their use.
// Every Q, dO or transposed operand a wave reads from LDS feeds two MFMAs (one per key tile).
//
// Pipeline of a step: the first GEMMs (S, dP) of the step, with the next step's tile transfers
// issued among them in four stages (one per MFMA, in the MFMAs' shadow); then 32 slots, each issuing
// one second-GEMM MFMA of the previous step (dV += P^T dO, dK += dS^T Q) beside part of this step's
// softmax (P, dS on the VALU), so that one wave keeps the matrix core busy while it computes P and dS.
// One barrier per step guards the tile buffers; the last four second-GEMM MFMAs of a step wait until
// after it, and run while the next step's first LDS reads are in flight.
#pragma once
#include "fa_bwd_kernels.hpp"

namespace fa {

struct Dkdv64Cfg {
  static constexpr int D = 128;                 // head dim of Q, K, V, dO
  static constexpr int KS = D / 16;             // MFMA k-steps over the head dim
  static constexpr int NTD = D / 32;            // 32-wide output tiles over the head dim
  static constexpr int QS = D + 8;              // padded row stride (elements) of the LDS tiles
  static constexpr int CPR = QS / 8;            // 16-byte chunks per padded row
  static constexpr int NW = 4, NT = 64 * NW;    // one wave per SIMD
  static constexpr int KPW = 64;                // keys per wave: two 32-key tiles
  static constexpr int BN = NW * KPW;           // keys per workgroup
  static constexpr int BM = 32;                 // query rows per step
  static constexpr int NBUF = 3;                // Q/dO buffers: steps i, i + 1 read, step i + 2 loading
  static constexpr int PF_A = 4;                // first GEMMs: LDS operands read this many MFMAs ahead
  static constexpr int PF_B = 2;                // second GEMMs: B fragments read this many pairs ahead
  static constexpr int MID_AT = 8;              // first-GEMM MFMA before which the next tile's loads issue
  static constexpr int DEFER = 4;               // second-GEMM MFMAs of a step issued after its barrier
  static constexpr int T_BYTES = (BM * QS * 2 + 1023) / 1024 * 1024;  // one Q (dO) buffer, whole 1 KB transfers
  static constexpr int NDMA = T_BYTES / 1024;
  static constexpr int NJ = (NDMA + NW - 1) / NW;  // transfers per wave per tile
  static constexpr int V_BYTES = BN * QS * 2;
  static constexpr int NDMA_V = V_BYTES / 1024;
  // the buffers read through per-step base registers come first, below the 64 KiB reach of the LDS
  // instructions' immediate offsets; the V and K tiles (per-lane base registers) follow
  static constexpr int OFF_Q = 0;                           // Q [NBUF][BM][QS]
  static constexpr int OFF_DO = OFF_Q + NBUF * T_BYTES;     // dO [NBUF][BM][QS]
  static constexpr int OFF_ST = OFF_DO + NBUF * T_BYTES;    // [NBUF][lse2, D][BM] fp32, MFMA row order
  static constexpr int OFF_V = (OFF_ST + NBUF * 2 * BM * 4 + 1023) / 1024 * 1024;  // V [BN][QS], 1 KB aligned
  // K: features 0 .. KREG*16 - 1 in registers, the rest in an LDS tile [BN][KH + 8]
  static constexpr int KREG = 4;                            // k-steps of S whose K fragments sit in registers
  static constexpr int KH = D - 16 * KREG;                  // features of K kept in LDS
  static constexpr int KHS = KH + 8;                        // padded row stride (elements) of that tile
  static constexpr int OFF_KH = OFF_V + V_BYTES;
  static constexpr int LDS_BYTES = OFF_KH + BN * KHS * 2;
  static_assert(V_BYTES % 1024 == 0 && T_BYTES % 1024 == 0, "tiles are whole 1 KB transfers");
  static_assert(LDS_BYTES % 16 == 0 && LDS_BYTES <= 160 * 1024, "LDS budget of one workgroup per CU");
  static_assert(OFF_KH % 16 == 0 && OFF_V % 1024 == 0 && KH % 16 == 0, "aligned tiles");
  static_assert(OFF_V <= 65536, "step buffers within the immediate-offset reach");
};

// DS: also store each step's dS (bf16) as one 16 KB block of the stored-dS form (fa_bwd_dqds.hpp), in the
// order the lanes hold the values: wave w's piece 2 n + s2 (1 KB) holds lane l's 16 bytes at 16 l.
template <bool CAUSAL, bool DS, bool WINDOW>
__global__ __attribute__((amdgpu_flat_work_group_size(Dkdv64Cfg::NT, Dkdv64Cfg::NT), amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkdv64(MainArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Dkdv64Cfg;
  constexpr int BN = C::BN, BM = C::BM, QS = C::QS, D = C::D, KS = C::KS, NTD = C::NTD;
  static_assert(CAUSAL || !WINDOW, "a window implies the causal bound");
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  float* s_st = (float*)(smem + C::OFF_ST);

  // work item: a host schedule names (kv tile, sequence * Hk + K/V head); the dense grid runs the heavy
  // (low) kv tiles first, tile-major over the heads and sequences, or head-major per XCD
  const int HB = a.Hk * a.batch;
  int tile, hb;
  if (a.sched) {
    tile = a.sched[2 * blockIdx.x];
    hb = a.sched[2 * blockIdx.x + 1];
  } else if (a.head_major) {  // HB % 8 == 0 (host): a bijection of the grid
    const int n_kt_max = (a.max_seqlen_kv + BN - 1) / BN;
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int kq = slot / n_kt_max;
    tile = slot - kq * n_kt_max;
    hb = x + 8 * kq;
  } else {
    tile = blockIdx.x / HB;
    hb = blockIdx.x - tile * HB;
  }
  const int b = hb / a.Hk, hk = hb - (hb / a.Hk) * a.Hk;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int kv0 = tile * BN;
  if (kv0 >= Lk) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int64_t rsq = (int64_t)a.H * D, rskq = (int64_t)a.Hk * D;  // row strides of Q/dO and of K/V
  const int rsqb = (int)(rsq * 2), rskqb = (int)(rskq * 2);
  const int G = a.H / a.Hk;

  {  // zero the tile buffers once: rows a transfer leaves untouched then hold finite values
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < C::OFF_KH; o += C::NT * 16) *(u32x4*)(smem + o) = z;
  }
  __syncthreads();

  // the steps: for each query head of the group, the 32-row q tiles that can see these keys
  // (window: query rows up to kv0 + BN - 1 + window - 1 see a key of the tile; the sum stays below 2^31,
  // as positions and the window, clamped to the longest sequence, stay below 2^30)
  const int n_qt = WINDOW ? imin((Lq + BM - 1) / BM, (kv0 + BN - 2 + a.window) / BM + 1) : (Lq + BM - 1) / BM;
  const int qt0 = CAUSAL ? kv0 / BM : 0;
  const int nq = n_qt > qt0 ? n_qt - qt0 : 0;
  const int n_steps = G * nq;
  // a step's position: q tile and query head, the byte offset of its Q (and dO) rows from the tensors'
  // bases, the index of its head's first statistic and (storing dS) the element offset of its dS block;
  // advanced one step at a time with additions
  struct Pos {
    int tile, head;
    int64_t off, srow, ds;
  };
  const int64_t head_off = (int64_t)(q_start + qt0 * BM) * rsqb;  // of the first step of a head, less the head
  constexpr int64_t DS_BLOCK = 256 * 32;
  auto advance = [&](Pos p) {
    p.off += BM * rsqb;
    p.ds += DS_BLOCK;
    if (++p.tile == qt0 + nq) {
      p.tile = qt0;
      ++p.head;
      p.off = head_off + (int64_t)p.head * (D * 2);
      p.srow += a.total_q;
      p.ds += ((int64_t)a.ds_nkt * a.ds_nqs - nq) * DS_BLOCK;  // the next head's block of this kv tile
    }
    return p;
  };

  const int kv_rows = imin(Lk - kv0, BN);
  const bf16* kbase = a.k + (kv_start + kv0) * rskq + (int64_t)hk * D;
  const bf16* vbase = a.v + (kv_start + kv0) * rskq + (int64_t)hk * D;
  // K fragments of this wave's keys: key 64 w + 32 n + c, features 16 ks + 8 hh .. + 7 (zero past Lk);
  // the first KREG k-steps in registers, the others in the LDS tile (each wave writes its own keys)
  constexpr int KREG = C::KREG;
  bf16x8 kreg[2][KREG];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, (int64_t)kv_rows * rskqb);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int ks = 0; ks < KREG; ++ks)
        kreg[n][ks] = __builtin_bit_cast(bf16x8, buf_load16(rk, (64 * w + 32 * n + c) * rskqb + (16 * ks + 8 * hh) * 2));
#pragma unroll
      for (int ks = KREG; ks < KS; ++ks) {
        const u32x4 x = buf_load16(rk, (64 * w + 32 * n + c) * rskqb + (16 * ks + 8 * hh) * 2);
        *(u32x4*)(smem + C::OFF_KH + ((64 * w + 32 * n + c) * C::KHS + 16 * (ks - KREG) + 8 * hh) * 2) = x;
      }
    }
  }
  {  // the V tile, once
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, (int64_t)kv_rows * rskqb);
    for (int j = w; j < C::NDMA_V; j += C::NW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(smem + C::OFF_V + 1024 * j),
                                               16, tile_dma_off(j, lane, C::CPR, rskqb, D), 0, 0, 0);
  }
  // Q and dO tile of a step into buffer bi: 9 transfers of 1 KB each, transfers w and w + 4 of every
  // wave and transfer 8 of wave 3 (wave 0 loads the statistics; the per-lane global offsets are formed
  // once). The work is issued in stages, one per first-GEMM MFMA, so that it runs in their shadow:
  // stage 0 forms the buffer resources, stages 1-3 issue the transfers and the statistics load.
  static_assert(C::NDMA == 9 && C::NW == 4 && 2 * BM == 64, "transfer and statistics assignment");
  const int dmo0 = tile_dma_off(w, lane, C::CPR, rsqb, D), dmo1 = tile_dma_off(w + 4, lane, C::CPR, rsqb, D);
  const int dmo2 = tile_dma_off(8, lane, C::CPR, rsqb, D);
  constexpr int kTileStages = 4;
  struct TileRsrc {
    __amdgpu_buffer_rsrc_t q, d;
  };
  auto tile_rsrc = [&](const Pos& ps) {
    // bytes of the tile's rows inside the sequence (below 2^31: 128 rows of a tensor span less than 2^30)
    const int n = imin(Lq - ps.tile * BM, BM) * rsqb;
    return TileRsrc{__builtin_amdgcn_make_buffer_rsrc((char*)a.q + ps.off, (short)0, n, kRsrcWord3),
                    __builtin_amdgcn_make_buffer_rsrc((char*)a.dout + ps.off, (short)0, n, kRsrcWord3)};
  };
  // untracked by the compiler: the step's first LDS reads of another buffer must not wait for it
  // (wait_tiles and the step's barrier order it before buffer bi is read)
  auto dma = [&](const TileRsrc& r, int bi, int j, int off) {
    dma16_untracked(r.q, off, (__attribute__((address_space(3))) void*)(smem + C::OFF_Q + bi * C::T_BYTES + 1024 * j));
    dma16_untracked(r.d, off, (__attribute__((address_space(3))) void*)(smem + C::OFF_DO + bi * C::T_BYTES + 1024 * j));
  };
  // row statistics of a step in MFMA row order, as the starting values of the S and dP accumulators:
  // lanes 0..31 of wave 0 store -lse2 / (scale log2 e), so that P = exp2(S_acc * scale * log2 e); lanes
  // 32..63 store -D, so that dS = P * dP_acc. Rows past the sequence get lse2 = +inf: their S starts at
  // -inf and their P (and dS) is exactly 0. The load reads a row inside the sequence (the last one for
  // rows past it) and the store replaces what such rows read.
  const float* const sbase = lane < BM ? a.lse2 : a.dvec;
  const int srow_lane = tile_row(lane & 31);
  auto load_stats = [&](const Pos& ps) -> float {
    const int r = imin(ps.tile * BM + srow_lane, Lq - 1);
    return sbase[ps.srow + r];
  };
  const float inv_sl2 = 1.f / a.scale_log2;
  auto store_stats = [&](int bi, float v, const Pos& ps) {
    if (w == 0) {
      const bool in_seq = ps.tile * BM + srow_lane < Lq;
      s_st[bi * 2 * BM + lane] = lane < BM ? (in_seq ? -(v * inv_sl2) : -__builtin_inff()) : (in_seq ? -v : -0.f);
    }
  };
  // piece e = 2 n + s2 of this wave's part of a step's dS block: this lane's 16 bytes (key 64 w + 32 n + c,
  // positions 16 hh + 8 s2 ..+7), non-temporal: the blocks are read once, by the dQ pass
  auto store_ds = [&](const Pos& ps, const bf16x8 (&d)[2][2], int e) {
    if constexpr (DS) {
      if (ps.tile >= a.ds_nqs || tile >= a.ds_nkt) return;  // outside the workspace (lengths past the maxima)
      const int n = e >> 1, s2 = e & 1;
      __builtin_nontemporal_store(d[n][s2], (bf16x8*)(a.ds + ps.ds + (w * 4 + e) * 512 + lane * 8));
    }
  };
  // stage k of the transfers of step ps into buffer bi (and of its statistics into st)
  auto issue_stage = [&](int k, const Pos& ps, int bi, TileRsrc& r, float& st) {
    if (k == 0) r = tile_rsrc(ps);
    if (k == 1) dma(r, bi, w, dmo0);
    if (k == 2) dma(r, bi, w + 4, dmo1);
    if (k == 3) {
      if (w == 3) dma(r, bi, 8, dmo2);
      if (w == 0) st = load_stats(ps);
    }
  };
  auto issue_tile = [&](const Pos& ps, int bi, float& st) {
    TileRsrc r;
#pragma unroll
    for (int k = 0; k < kTileStages; ++k) issue_stage(k, ps, bi, r, st);
  };

  // The dK, dV sums stay in the accumulator registers (AGPRs) for the whole kernel, and the S/dP
  // accumulators, which the softmax reads, in the vector registers: the compiler gives one register
  // file to all MFMAs of a kernel, so the dK/dV MFMAs are written as inline assembly on AGPR operands.
  // The compiler's hazard checks do not look inside an asm statement: an MFMA must not read a register
  // (A, B or the accumulator) that a VALU instruction wrote fewer than two wait states before, and the
  // register allocator may place such a write, an AGPR copy when it moves a sum to another tuple,
  // directly before one. Inside the step loop the operands are written a step ahead and the sums stay
  // in place; at the loop's exit the allocator may move sums, so the last step's MFMAs carry the two
  // wait states themselves (guarded). Same-register accumulation chains need none; the read of the
  // sums after the last MFMA waits explicitly (before the write-back).
  auto mfma_acc = [](auto guarded, f32x16& acc, const bf16x8& x, const bf16x8& y) {
    if constexpr (decltype(guarded)::value)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
  };
  f32x16 accV[2][NTD], accK[2][NTD];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int nt = 0; nt < NTD; ++nt) {
      accV[n][nt] = f32x16{};
      accK[n][nt] = f32x16{};
    }

  const int arow = tile_row(c) * QS + 8 * hh;                                 // A rows of the Q, dO tiles
  const int vrow = (64 * w + c) * QS + 8 * hh;                                // B rows of V (key tile 0)
  const int brow = (hh + 4 * (gi >> 2)) * QS + 16 * (g & 1) + 4 * (gi & 3);  // transposed B reads
  // LDS operands are addressed through address-space-3 pointers, so that the constant part of each
  // offset folds into the instruction's immediate field
  typedef __attribute__((address_space(3))) const bf16 lds_bf16;
  lds_bf16* const L = (lds_bf16*)smem;
  auto tq = [&](int bi) { return L + (C::OFF_Q + bi * C::T_BYTES) / 2; };
  auto tdo = [&](int bi) { return L + (C::OFF_DO + bi * C::T_BYTES) / 2; };
  // a per-lane base register: the constant offsets added to it then fit the immediate field
  auto base = [](lds_bf16* p) {
    asm volatile("" : "+v"(p));
    return p;
  };
  auto rd16 = [](lds_bf16* p) { return *(const __attribute__((address_space(3))) bf16x8*)p; };
  auto rd_tr = [](lds_bf16* p) {
    return concat(__builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p)),
                  __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 2 * QS))));
  };

  // every key of this wave visible from every row of step sp: no element mask (wave-uniform)
  auto full_step = [&](int qtile) {
    return (!CAUSAL || kv0 + 64 * w + 63 <= qtile * BM) && (!WINDOW || qtile * BM + BM - 1 - (kv0 + 64 * w) < a.window);
  };
  // First GEMMs of step sp over buffer bi: S = Q K^T for both key tiles over the 8 k-steps, then
  // dP = dO V^T; each Q or dO fragment feeds both key tiles. Operands are read PF MFMAs ahead. The
  // accumulators start from the row statistics (above); under a causal mask, on steps whose rows do
  // not see every key of the wave, S of an invisible (row, key) pair starts at -inf instead, so that
  // its P is exactly 0. Element (a4, bb) of a lane is MFMA row 8 a4 + 4 hh + bb = tile row
  // hh + 2 (a4 % 2) + 4 bb + 16 (a4 / 2); key kv0 + 64 w + 32 n + c is visible from query row
  // i0 + r iff kv0 + 64 w + c - i0 - hh <= r - hh - 32 n, a constant right side per element.
  auto gemm1 = [&](int qtile, int bi, f32x16 (&s)[2], f32x16 (&dp)[2], auto&& mid, auto&& pre) {
    constexpr int PF = C::PF_A;
    lds_bf16* sq = base(tq(bi) + arow);
    lds_bf16* sd = base(tdo(bi) + arow);
    const float* st = s_st + bi * 2 * BM;
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      l4[a4] = *(const f32x4*)(st + 8 * a4 + 4 * hh);
      d4[a4] = *(const f32x4*)(st + BM + 8 * a4 + 4 * hh);
    }
    bf16x8 qf[KS], df[KS], vf[KS][2], kf[KS][2];
    lds_bf16* s_kh = base(L + C::OFF_KH / 2 + (64 * w + c) * C::KHS + 8 * hh);
    lds_bf16* s_vw = base(L + C::OFF_V / 2 + vrow);
    // MFMA m: k-step ks = m / 4, then S of key tile 0, S of tile 1, dP of tile 0, dP of tile 1 (four
    // independent accumulation chains)
    auto load_op = [&](int m) {
      if (m >= 32) return;
      const int ks = m >> 2, n = m & 1;
      if ((m & 2) == 0) {
        if (n == 0) qf[ks] = rd16(sq + 16 * ks);
        if (ks >= KREG) kf[ks][n] = rd16(s_kh + 32 * n * C::KHS + 16 * (ks - KREG));
      } else {
        if (n == 0) df[ks] = rd16(sd + 16 * ks);
        vf[ks][n] = rd16(s_vw + 32 * n * QS + 16 * ks);
      }
    };
#pragma unroll
    for (int m = 0; m < PF; ++m) load_op(m);
    __builtin_amdgcn_sched_barrier(0);
    pre();  // MFMAs that need none of these reads run while they are in flight
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s_init[2], dp_init;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        s_init[0][4 * a4 + bb] = l4[a4][bb];
        dp_init[4 * a4 + bb] = d4[a4][bb];
      }
    s_init[1] = s_init[0];
    if (!full_step(qtile)) {
      // opaque to the optimiser, so that the 32 comparisons stay against immediates inside the loop
      // instead of becoming per-element values held across it. Window: the key is too old for the
      // row iff kv0 + 64 w + 32 n + c <= row - window, i.e. t + window <= (the same right side).
      int t = kv0 + 64 * w + c - qtile * BM - hh;
      asm volatile("" : "+v"(t));
      int tw = 0;
      if constexpr (WINDOW) {
        tw = t + a.window;
        asm volatile("" : "+v"(tw));
      }
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const int rhs = 2 * (a4 & 1) + 4 * bb + 16 * (a4 >> 1) - 32 * n;
            if (t > rhs || (WINDOW && tw <= rhs)) s_init[n][4 * a4 + bb] = -__builtin_inff();
          }
    }
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      load_op(m + PF);
      // the next step's loads (and, storing dS, the previous step's four dS pieces first), in the MFMAs'
      // shadow
      if (m >= C::MID_AT - (DS ? 4 : 0) && m < C::MID_AT + kTileStages) {
        __builtin_amdgcn_sched_barrier(0);
        mid(m - C::MID_AT);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int ks = m >> 2, n = m & 1;
      if ((m & 2) == 0)
        s[n] = mfma32x32x16(qf[ks], ks < KREG ? kreg[n][ks < KREG ? ks : 0] : kf[ks][n], ks == 0 ? s_init[n] : s[n]);
      else
        dp[n] = mfma32x32x16(df[ks], vf[ks][n], ks == 0 ? dp_init : dp[n]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // 32 slots: slot m issues the second-GEMM MFMA m of the previous step (buffer bq; P, dS in pk0, dsk0)
  // and softmax element m of the current step (S, dP in s, dp) into pk1, dsk1, so that the VALU work
  // of one step runs beside the matrix work of the previous one.
  //  - second GEMMs: MFMA m uses B fragment i = m / 2 (i < 8: dO^T for dV += P^T dO, then Q^T for
  //    dK += dS^T Q; k-step s2 = i / 4 % 2, output tile nt = i % 4) for key tile n = m % 2. k-step s2's
  //    k-index e is MFMA row 16 s2 + 4 hh + e (e < 4) or 16 s2 + 8 + 4 hh + e - 4; the transposed reads
  //    fetch those tile rows;
  //  - softmax: key tile n = m / 16 first (tile 0's S and dP registers are free for the second half),
  //    element j = m % 16: P = exp2(S_acc * scale * log2 e), dS = P * dP_acc (the accumulators
  //    started from the statistics).
  //  - beside a softmax (inside the loop), the last DEFER MFMAs are left to the next step, which issues
  //    them after the barrier while its first LDS reads are in flight; their B fragments go to bfd.
  constexpr int ND = C::DEFER, NDB = ND / 2 > 0 ? ND / 2 : 1;
  static_assert(ND % 2 == 0 && ND <= 16, "deferred MFMAs come in key-tile pairs of the dK part");
  auto slots = [&](auto with_g2, auto with_sm, int bq, const f32x16 (&s)[2], const f32x16 (&dp)[2],
                   const bf16x8 (&pk0)[2][2], const bf16x8 (&dsk0)[2][2], bf16x8 (&pk1)[2][2],
                   bf16x8 (&dsk1)[2][2], bf16x8 (&bfd)[NDB]) {
    constexpr bool G2 = decltype(with_g2)::value, SM = decltype(with_sm)::value;
    constexpr int PFB = C::PF_B;
    lds_bf16* sq = base(tq(bq) + brow);
    lds_bf16* sd = base(tdo(bq) + brow);
    bf16x8 bf[16];
    auto load_b = [&](int i) {
      if (i >= 16) return;
      const int part = i >> 3, s2 = (i >> 2) & 1, nt = i & 3;
      bf[i] = rd_tr((part == 0 ? sd : sq) + 16 * s2 * QS + 32 * nt);
    };
    // the softmax of element e is spread over three slots, so that the instructions a slot issues
    // are independent of each other: slot m scales element m + 2, exponentiates element m + 1 and
    // forms dS of element m (and packs P, dS of the element pair ending at m)
    // Each result is pinned to its slot by an empty asm statement that takes it as an operand: the
    // values are only needed one step later, and without the pins the optimiser sinks the whole
    // softmax below the MFMAs of the step.
    float xs[32], ps[32];
    auto sm_scale = [&](int e) {
      if (e < 32) {
        xs[e] = s[e >> 4][e & 15] * a.scale_log2;
        asm volatile("" : "+v"(xs[e]));
      }
    };
    auto sm_exp = [&](int e) {
      if (e < 32) {
        ps[e] = fast_exp2(xs[e]);
        asm volatile("" : "+v"(ps[e]));
      }
    };
    auto sm_elem = [&](int m) {
      const int n = m >> 4, j = m & 15;
      pk1[n][j >> 3][j & 7] = to_bf16(ps[m]);
      dsk1[n][j >> 3][j & 7] = to_bf16(ps[m] * dp[n][j]);
      if (j & 1) asm volatile("" : "+v"(pk1[n][j >> 3]), "+v"(dsk1[n][j >> 3]));
    };
    if constexpr (G2) {
#pragma unroll
      for (int i = 0; i < PFB; ++i) load_b(i);
    }
    if constexpr (SM) {
      sm_scale(0);
      sm_scale(1);
      sm_exp(0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      if constexpr (G2) {
        if ((m & 1) == 0) load_b((m >> 1) + PFB);
        const int i = m >> 1, n = m & 1, part = i >> 3, s2 = (i >> 2) & 1, nt = i & 3;
        // the last step (no softmax beside it) follows the loop's exit
        constexpr std::bool_constant<!SM> guarded{};
        if (SM && m >= 32 - ND) {
          if (n == 0) bfd[i - (16 - NDB)] = bf[i];
        } else if (part == 0) {
          mfma_acc(guarded, accV[n][nt], pk0[n][s2], bf[i]);
        } else {
          mfma_acc(guarded, accK[n][nt], dsk0[n][s2], bf[i]);
        }
      }
      if constexpr (SM) {
        sm_scale(m + 2);
        sm_exp(m + 1);
        sm_elem(m);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the MFMAs a step left over (dK += dS^T Q of its last output tiles), from the dS registers dsk0
  auto deferred = [&](auto guarded, const bf16x8 (&bfd)[NDB], const bf16x8 (&dsk0)[2][2]) {
    if constexpr (ND > 0) {
#pragma unroll
      for (int m = 32 - ND; m < 32; ++m) {
        const int i = m >> 1, n = m & 1, s2 = (i >> 2) & 1, nt = i & 3;
        mfma_acc(guarded, accK[n][nt], dsk0[n][s2], bfd[i - (16 - NDB)]);
      }
    }
  };
  auto wait_tiles = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x16 s[2], dp[2];
  bf16x8 pk[2][2], dsk[2][2], pkn[2][2], dskn[2][2], bfd[NDB];
  if (n_steps > 0) {
    // prologue: tiles of steps 0 and 1 in flight; the first GEMMs and the softmax of step 0
    float st0 = 0.f, st1 = 0.f;
    Pos cur = {qt0, hk * G, head_off + (int64_t)hk * G * (D * 2), (int64_t)hk * G * a.total_q + q_start,
               DS ? (((int64_t)(b * a.H + hk * G) * a.ds_nkt + tile) * a.ds_nqs + qt0) * DS_BLOCK : 0};  // step 0
    Pos nxt = advance(cur);  // step 1
    issue_tile(cur, 0, st0);
    if (n_steps > 1) issue_tile(nxt, 1, st1);
    wait_tiles();
    store_stats(0, st0, cur);
    if (n_steps > 1) store_stats(1, st1, nxt);
    __syncthreads();
    gemm1(cur.tile, 0, s, dp, [](int) {}, [] {});
    slots(std::false_type{}, std::true_type{}, 0, s, dp, pkn, dskn, pk, dsk, bfd);
    // the first step's deferred MFMAs (it has none) add zero products
#pragma unroll
    for (int i = 0; i < NDB; ++i) bfd[i] = bf16x8{};
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int e = 0; e < 2; ++e) dskn[n][e] = bf16x8{};
    // step sp: the tile of sp + 1 loads; the first GEMMs of sp, then the second GEMMs of sp - 1 beside
    // the softmax of sp
    int bq = 0, bp = 0, b1 = 1;  // buffers of steps sp - 1, sp, sp + 1 (rotating through NBUF)
    auto step = [&](int sp, const bf16x8 (&pko)[2][2], const bf16x8 (&dsko)[2][2], bf16x8 (&pkw)[2][2],
                    bf16x8 (&dskw)[2][2]) {
      const Pos prv = cur;
      cur = nxt;
      nxt = advance(cur);
      bq = bp;
      bp = b1;
      b1 = b1 == C::NBUF - 1 ? 0 : b1 + 1;
      float st2 = 0.f;
      const bool has1 = sp + 1 < n_steps;
      TileRsrc rn;
      // the previous step's deferred MFMAs read the dS registers this step's softmax rewrites
      gemm1(cur.tile, bp, s, dp, [&](int k) {
        if (k < 0)
          store_ds(prv, dsko, k + 4);
        else if (has1)
          issue_stage(k, nxt, b1, rn, st2);
      }, [&] { deferred(std::false_type{}, bfd, dskw); });
      slots(std::true_type{}, std::true_type{}, bq, s, dp, pko, dsko, pkw, dskw, bfd);
      if (has1) store_stats(b1, st2, nxt);
      wait_tiles();
      __syncthreads();
    };
    // two steps per iteration, the P and dS registers of one step and the next swapping roles
    int sp = 1;
    for (; sp + 1 < n_steps; sp += 2) {
      step(sp, pk, dsk, pkn, dskn);
      step(sp + 1, pkn, dskn, pk, dsk);
    }
    if (sp < n_steps) {  // then P, dS of the last step in pk, dsk and those of the step before in pkn, dskn
      step(sp, pk, dsk, pkn, dskn);
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const bf16x8 tp = pk[n][e], td = dsk[n][e];
          pk[n][e] = pkn[n][e];
          dsk[n][e] = dskn[n][e];
          pkn[n][e] = tp;
          dskn[n][e] = td;
        }
    }
    // the last step's deferred MFMAs (the step before it in dskn), after the loop's exit
    deferred(std::true_type{}, bfd, dskn);
#pragma unroll
    for (int e = 0; e < 4; ++e) store_ds(cur, dsk, e);  // the last step's dS
    // epilogue: the second GEMMs of the last step
    slots(std::true_type{}, std::false_type{}, bp, s, dp, pk, dsk, pkn, dskn, bfd);
  }

  // the last accumulating MFMA has written the sums before they are read (more than the 18 wait
  // states the longest MFMA needs)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // write-back of keys kv0 + 64 w + 32 n + 8 a + 4 hh + b, features 32 nt + c: dV, and dK = scale * acc
#pragma unroll
  for (int n = 0; n < 2; ++n) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int r = kv0 + 64 * w + 32 * n + 8 * a4 + 4 * hh + bb;
        if (r < Lk) {
          const int64_t o = (kv_start + r) * rskq + (int64_t)hk * D + c;
#pragma unroll
          for (int nt = 0; nt < NTD; ++nt) {
            a.dv[o + 32 * nt] = to_bf16(accV[n][nt][4 * a4 + bb]);
            a.dk[o + 32 * nt] = to_bf16(accK[n][nt][4 * a4 + bb] * a.scale);
          }
        }
      }
    }
  }
#endif
}

}  // namespace fa
