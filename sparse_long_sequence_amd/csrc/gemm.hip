// Encoder-layer GEMMs on the gfx950 matrix cores, with fused epilogues, and the
// LayerNorm row kernel.
//
// [FT-LF] = the page "FasterTransformer Longformer 推理加速实践：PyTorch 集成、输入约束与
// 端到端性能解析", section "Longformer Encoder 计算流程", per-layer steps:
//   1  the Q / K / V / global-K / global-V projections (one packed GEMM) and the
//      global-query projection of the leading G tokens, bias added and the result
//      split into heads;                                  -> epilogue kEpiHeads
//   5  attention output projection + bias + residual, then LayerNorm
//                                                         -> kEpiResidT + layernorm
//   6  FFN: GEMM + bias + GELU, GEMM + bias + residual, then LayerNorm
//                                                         -> kEpiGelu, kEpiResidF32
// (steps 3-4, the attention itself, are attn_mfma.hip).
//
// C[m, n] = sum_k A[arow(m), k] * W[n, k] + bias[n]: both operands are read as rows
// of consecutive k, which is the operand layout of v_mfma_f32_32x32x16 (lane (n, g)
// holds 8 consecutive k of one row).  The weight rows are the MFMA's first operand
// and the activation rows its second, so each lane's 16 accumulators are 4 groups
// of 4 consecutive output columns of ONE output row: the epilogue stores 8-byte
// runs.  Two tile shapes of one kernel: 256 x 256 with 8 waves of 128 x 64 (4 x 2
// MFMA tiles, 6 fragment reads per 8 MFMAs) for GEMMs whose grid still covers every
// CU, else 128 x 128 with 4 waves of 64 x 64 (two workgroups per CU).  K step 64;
// the operand tiles go from global memory straight into LDS (buffer_load_dwordx4 ...
// lds: lane L of a wave's load lands at LDS base + 16 L, every lane's global address
// is free), double-buffered, so there is no register staging and no LDS store
// phase: each K step issues the next step's loads into the other buffer, multiplies
// the current one, waits for this wave's loads and meets the others at a barrier.
// Rows of A past M read out of range (zeros) and are not stored.
#include <type_traits>

#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

namespace {

constexpr int kGT = 128;      // smallest tile: N must be a multiple of it
constexpr int kGK = 64;       // K step
constexpr int kGroupM = 8;    // m-tiles per group of the tile order (L2 reuse of W tiles)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// The erf form of GELU ([FT-LF] step 6 names GELU; the exact form is the reading),
// x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), with erf from Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26: for z >= 0,
// erf z = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2), t = 1 / (1 + p z),
// absolute error at most 1.5e-7; erf is odd.  About a dozen vector instructions,
// against several dozen for the library erff, which dominated the FFN1 epilogue.
__device__ inline float gelu(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);
  const float erf_abs = fmaf(-poly, e, 1.0f);
  const float erf_x = __builtin_copysignf(erf_abs, x);
  return 0.5f * x * (1.0f + erf_x);
}

// Residual operand of the residual epilogues (4 columns of one row, as stored).
template <typename T, int EPI> struct ResidVec { typedef typename Elem<T>::vec4 type; };
template <typename T> struct ResidVec<T, kEpiResidF32> { typedef f32x4 type; };

// Epilogue of 4 consecutive output columns nb .. nb + 3 of row m (acc = the raw sums,
// bv = their bias, rv = their residual; GELU and residual epilogues).
template <typename T, int EPI>
__device__ __forceinline__ void epilogue4(const GemmArgs& g, int m, int nb, const float acc[4],
                                          const typename Elem<T>::vec4& bv,
                                          const typename ResidVec<T, EPI>::type& rv) {
  typedef typename Elem<T>::vec4 v4;
  float r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = acc[e] + Elem<T>::to_f(bv[e]);
  if (EPI == kEpiGelu) {
    v4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = Elem<T>::from_f(gelu(r[e]));
    *(v4*)((T*)g.out + (size_t)m * g.ldo + nb) = w;
  } else {
    f32x4 z;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      z[e] = r[e] + (EPI == kEpiResidF32 ? (float)rv[e] : Elem<T>::to_f(rv[e]));
    *(f32x4*)((float*)g.out + (size_t)m * g.ldo + nb) = z;
  }
}

// Stores of 16-bit outputs w[jj] = columns 8 jj + 4 gq .. + 3 of one row (jj = 0..3;
// dst = the row's column 0 of the 32-column tile): lanes n and n + 32 hold the two
// halves of each 8-column group and send each other the half the other lacks (every
// lane of the pair active), so lane gq stores columns 16 p + 8 gq .. + 7 (p = 0, 1) as
// one 16-byte store: half the store instructions of 8-byte stores.
template <typename T>
__device__ __forceinline__ void store_pairs16(T* dst, int gq, const typename Elem<T>::vec4 w[4]) {
  static_assert(sizeof(T) == 2, "16-bit outputs");
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const u32x2 x = __builtin_bit_cast(u32x2, w[2 * p]), y = __builtin_bit_cast(u32x2, w[2 * p + 1]);
    const u32x2 sd = gq ? x : y;
    const u32x2 rb = {(uint32_t)__shfl_xor((int)sd[0], 32), (uint32_t)__shfl_xor((int)sd[1], 32)};
    *(u32x4*)(dst + 16 * p + 8 * gq) = gq ? u32x4{rb[0], rb[1], y[0], y[1]} : u32x4{x[0], x[1], rb[0], rb[1]};
  }
}

// Epilogue of one 32 x 32 MFMA tile: the lane's 16 sums are columns cbase + 8 jj +
// 4 gq .. + 3 (jj = 0..3) of output row m, with their bias bv[jj] and residual
// rv[jj] already in registers; cbase (a multiple of 32) is the same for the whole
// wave, and D is a multiple of 64, so for the head split the tensor and head come
// from cbase alone (one scalar division per tile, none per element).
template <typename T, int EPI>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& g, int m, int cbase, int gq,
                                              const f32x16& acc, int split,
                                              const typename Elem<T>::vec4 bv[4],
                                              const typename ResidVec<T, EPI>::type rv[4]) {
  typedef typename Elem<T>::vec4 v4;
  if (EPI == kEpiPartial) {
    float* dst = g.part + ((size_t)split * g.M + m) * g.N + cbase + 4 * gq;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      *(f32x4*)(dst + 8 * jj) = f32x4{acc[4 * jj], acc[4 * jj + 1], acc[4 * jj + 2], acc[4 * jj + 3]};
    return;
  }
  if (EPI == kEpiHeads) {
    const int ti = cbase / g.D, nn = cbase - ti * g.D;
    const int h = nn >> 6, d0 = nn & 63;
    const int bb = m / g.rows, rr = m - bb * g.rows;
    T* dst = (T*)g.heads[ti] + (((size_t)bb * g.H + h) * g.rows + rr) * 64 + d0;
    v4 w[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[jj][e] = Elem<T>::from_f(acc[4 * jj + e] + Elem<T>::to_f(bv[jj][e]));
    if constexpr (sizeof(T) == 2) {
      store_pairs16<T>(dst, gq, w);
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) *(v4*)(dst + 8 * jj + 4 * gq) = w[jj];
    }
    return;
  }
  if constexpr (EPI == kEpiGelu && sizeof(T) == 2) {
    v4 w[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[jj][e] = Elem<T>::from_f(gelu(acc[4 * jj + e] + Elem<T>::to_f(bv[jj][e])));
    store_pairs16<T>((T*)g.out + (size_t)m * g.ldo + cbase, gq, w);
    return;
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float r[4] = {acc[4 * jj], acc[4 * jj + 1], acc[4 * jj + 2], acc[4 * jj + 3]};
    epilogue4<T, EPI>(g, m, cbase + 8 * jj + 4 * gq, r, bv[jj], rv[jj]);
  }
}

__device__ inline int xcd_chunk(int i, int n) {
  // consecutive workgroup ids go round-robin over the 8 XCDs: give each XCD a
  // contiguous run of tile indices, so its workgroups share W tiles in its L2
  const int per = n / 8;
  const int full = per * 8;
  if (i >= full) return i;
  return (i % 8) * per + i / 8;
}

// Tile layout in LDS: rows of CH chunks of 16 B (8 k values each; CH = KS / 8), no
// padding; slot s of row r holds chunk s ^ swz(r).  The LDS serves a 16-byte read 16
// lanes at a time over 64 four-byte banks (measured on gfx950: a wave-wide
// ds_read_b128 costs 5.6 cycles when those 16 lanes cover all 64 banks, 8.0 with
// two-way conflicts), and a fragment read gives its 16 lanes 16 consecutive rows of
// one chunk.  With 128-byte rows (CH = 8) a row's bank groups are 8 (r & 1) + slot,
// so the slot must differ between the 8 even rows and between the 8 odd rows:
// swz(r) = (r >> 1) & 7.  With 64-byte rows (CH = 4) the groups are 4 (r & 3) +
// slot: swz(r) = (r >> 2) & 3.  Load i of wave w fills chunks (NL w + i) 64 + lane,
// i.e. row (64 / CH) (NL w + i) + lane / CH, slot lane % CH.
template <int CH>
__device__ inline int swz(int r) {
  return CH == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

template <typename T, int NL>
__device__ inline void dma_tile(rsrc_t r, const int off[NL], int kb, T* lds_tile, int wave) {
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
#pragma unroll
  for (int i = 0; i < NL; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(lds_tile + (wave * NL + i) * 64 * EPC), 16,
        off[i] < 0 ? -1 : off[i] + kb, 0, 0, 0);
}

// 16-byte MFMA operand fragment: 8 fp16 / bf16 values (one 32x32x16 MFMA) or 4 fp32
// values (four 32x32x2 MFMAs).
template <typename T> struct GemmFrag { typedef typename Elem<T>::vec8 type; };
template <> struct GemmFrag<float> { typedef f32x4 type; };

// Workgroup barrier without __syncthreads' release fence: that fence would wait for
// every load in flight (the direct-to-LDS loads count as pending LDS writes), which
// would drain the prefetch pipeline at every step.  Each step has already consumed
// all of its LDS reads (the MFMAs wait for them) and waited for the loads the next
// step reads; the empty asm keeps the compiler from moving memory accesses across.
__device__ inline void step_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt with only the vector-memory count set (expcnt and lgkmcnt left free).
template <int VM>
__device__ inline void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup tile TM x TN (rows of A x rows of W), WAVES waves of WM x WN each, K step
// KS, ST LDS stages: the loads of step ks + ST - 1 are issued at step ks.  The stages
// are separate LDS objects and the K loop is unrolled by ST steps, so every access
// names its stage statically: the compiler then knows that the loads in flight write
// other stages and does not make the current step's LDS reads wait for them.
//
// Second problem (head-split epilogue only): workgroups from tiles0 on take the tiles
// of g1, a GEMM of the same K and dtype, so a small GEMM rides in the idle slots of a
// large one's last round of tiles instead of a launch of its own.
template <typename T, int EPI, int TM, int TN, int WAVES, int WM, int WN, int KS, int ST>
__global__ __launch_bounds__(64 * WAVES) void gemm_kernel(GemmArgs g0, GemmArgs g1, int tiles0) {
  typedef typename GemmFrag<T>::type v8;
  constexpr int MI = WM / 32, NI = WN / 32;    // MFMA tiles per wave
  constexpr int WAVES_M = TM / WM;
  constexpr int EPC = 16 / (int)sizeof(T);     // elements per 16-byte chunk
  constexpr int CH = KS / EPC;                 // 16-byte chunks per tile row
  constexpr int RPL = 64 / CH;                 // tile rows per wave-wide load
  constexpr int NLA = TM / (RPL * WAVES), NLW = TN / (RPL * WAVES);   // loads per step
  constexpr int NL = NLA + NLW;
  constexpr int D = ST - 1;                    // prefetch distance in steps
  static_assert(WAVES_M * (TN / WN) == WAVES, "waves tile the workgroup tile");
  static_assert(NLA * RPL * WAVES == TM && NLW * RPL * WAVES == TN, "whole loads per wave");
  static_assert(CH == 4 || CH == 8, "K step 32 or 64");
  static_assert(ST >= 2 && ST <= 4 && (D - 1) * NL < 64, "stages");
  // one LDS object per stage (A tile, then W tile): the compiler tells in-flight
  // direct-to-LDS loads apart from later LDS reads by the object they write, and
  // only for a few objects, so the two tiles of a stage share one
  __shared__ __attribute__((aligned(16))) T st0[(TM + TN) * KS], st1[(TM + TN) * KS];
  __shared__ __attribute__((aligned(16))) T st2[ST > 2 ? (TM + TN) * KS : 8];
  __shared__ __attribute__((aligned(16))) T st3[ST > 3 ? (TM + TN) * KS : 8];
  auto abuf = [&](auto J) -> T* {
    constexpr int j = decltype(J)::value % ST;
    if constexpr (j == 0) return st0;
    else if constexpr (j == 1) return st1;
    else if constexpr (j == 2) return st2;
    else return st3;
  };
  auto wbuf = [&](auto J) -> T* { return abuf(J) + TM * KS; };
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n = lane & 31, gq = lane >> 5;
  const bool second = EPI == kEpiHeads && (int)blockIdx.x >= tiles0;
  // the problem's arguments read in place from the kernel-argument segment: the
  // AMDGPU kernel ABI lays the arguments out in order, each at its natural alignment,
  // so g0 sits at offset 0 and g1 at sizeof(GemmArgs) (a multiple of its alignment).
  // A select between the two parameters themselves would copy both to scratch memory.
  typedef __attribute__((address_space(4))) const GemmArgs* kargs_t;
  const GemmArgs& g =
      *(const GemmArgs*)((kargs_t)__builtin_amdgcn_kernarg_segment_ptr() + (second ? 1 : 0));
  const int bx = second ? (int)blockIdx.x - tiles0 : (int)blockIdx.x;

  // tile order: per XCD a contiguous run of tile indices; within it, groups of
  // kGroupM m-tiles sweep all n-tiles, so a W tile is reused while it is in L2; with
  // split-K the grid holds every tile once per split (the second problem's few tiles
  // keep their order)
  const int tiles_n = g.N / TN;
  const int tiles_m = (g.M + TM - 1) / TM;
  const int flat = second ? bx : xcd_chunk(bx, tiles_m * tiles_n * g.splits);
  const int split = __builtin_amdgcn_readfirstlane(flat / (tiles_m * tiles_n));
  const int bid = flat - split * (tiles_m * tiles_n);
  const int per_group = kGroupM * tiles_n;
  const int grp = bid / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(kGroupM, tiles_m - first_m);
  const int in_grp = bid - grp * per_group;
  const int tm = __builtin_amdgcn_readfirstlane(first_m + in_grp % gsize);
  const int tn = __builtin_amdgcn_readfirstlane(in_grp / gsize);
  const int m0 = tm * TM, n0 = tn * TN;

  const rsrc_t ra = make_rsrc(g.a, 0x7fffffff);
  const rsrc_t rw = make_rsrc(g.w, 0x7fffffff);
  const int lrow = lane / CH;
  // global chunk of this lane's 16 bytes in tile row r: the swizzle of that row
  auto lchunk = [&](int r) { return (lane % CH) ^ swz<CH>(r); };
  const int kspan = g.K / g.splits, k0 = split * kspan;
  int aoff[NLA], woff[NLW];
#pragma unroll
  for (int i = 0; i < NLA; ++i) {
    const int r = RPL * (NLA * wave + i) + lrow;
    const int m = m0 + r;
    int arow = m;
    if (g.a_group > 0 && m < g.M) {
      const int base = (m / g.a_group) * g.a_group_stride;
      arow = base + (g.a_rows ? g.a_rows[base + m % g.a_group] : m % g.a_group);
    }
    aoff[i] = m < g.M ? (arow * g.lda + k0 + EPC * lchunk(r)) * (int)sizeof(T) : -1;
  }
#pragma unroll
  for (int i = 0; i < NLW; ++i) {
    const int r = RPL * (NLW * wave + i) + lrow;
    woff[i] = ((n0 + r) * g.ldw + k0 + EPC * lchunk(r)) * (int)sizeof(T);
  }

  const int wm = (wave % WAVES_M) * WM, wn = (wave / WAVES_M) * WN;
  f32x16 acc[NI][MI];   // [n sub-tile][m sub-tile]
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j) acc[i][j] = f32x16{};

  // fragment of tile row rr (sub-tiles start at multiples of 32), chunk c
  auto frag = [&](const T* tile, int rr, int c) {
    return *(const v8*)(tile + (rr * CH + (c ^ swz<CH>(rr))) * EPC);
  };
  const int nk = kspan / KS;
  const int kstep = KS * (int)sizeof(T);
  auto issue = [&](auto J, int ks) {   // loads of step ks into stage J
    dma_tile<T, NLA>(ra, aoff, ks * kstep, abuf(J), wave);
    dma_tile<T, NLW>(rw, woff, ks * kstep, wbuf(J), wave);
  };
  // step ks (stage J = ks % ST): issue step ks + D into stage J + D, multiply stage J,
  // wait until step ks + 1 has landed (the D - 1 later steps may stay in flight), barrier
  auto step = [&](auto J, int ks) {
    constexpr int j = decltype(J)::value;
    if (ks + D < nk) issue(std::integral_constant<int, j + D>{}, ks + D);
    const T* ca = abuf(J);
    const T* cw = wbuf(J);
    // 256 x 256 tiles (8 MFMAs per round): fragments in two register sets, the reads
    // of round kk + 1 out before the MFMAs of round kk, so their latency hides behind
    // those MFMAs (1 % on the encoder layer; the smaller tiles were slower with it)
    constexpr int NKK = KS / (2 * EPC);   // rounds of two chunks (the g halves)
    constexpr bool kPipe = NI * MI >= 8;
    v8 wf[2][NI], xf[2][MI];
    auto read_round = [&](int kk, v8* w_, v8* x_) {
#pragma unroll
      for (int i = 0; i < NI; ++i) w_[i] = frag(cw, wn + 32 * i + n, 2 * kk + gq);
#pragma unroll
      for (int q = 0; q < MI; ++q) x_[q] = frag(ca, wm + 32 * q + n, 2 * kk + gq);
    };
    if constexpr (kPipe) {
      read_round(0, wf[0], xf[0]);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 1 < NKK) read_round(kk + 1, wf[(kk + 1) & 1], xf[(kk + 1) & 1]);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int q = 0; q < MI; ++q)
            acc[i][q] = mfma32(wf[kk & 1][i], xf[kk & 1][q], acc[i][q]);
      }
      // the order for the scheduler (it would otherwise sink each round's reads below
      // the previous round's MFMAs, into the same registers): rounds 0 and 1 read,
      // then per round its MFMAs followed by the next-but-one round's reads
      constexpr int RD = NI + MI;                                   // LDS reads per round
      constexpr int MF = NI * MI * (sizeof(T) == 4 ? 4 : 1);        // MFMAs per round
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * RD, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
        if (kk + 2 < NKK) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        read_round(kk, wf[0], xf[0]);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int q = 0; q < MI; ++q) acc[i][q] = mfma32(wf[0][i], xf[0][q], acc[i][q]);
      }
    }
    if (ks + D < nk) wait_vm<(D - 1) * NL>();
    else wait_vm<0>();
    step_barrier();
  };
  // prologue: steps 0 .. D - 1 in flight, step 0 landed
  issue(std::integral_constant<int, 0>{}, 0);
  if (D > 1 && 1 < nk) issue(std::integral_constant<int, 1>{}, 1);
  if (D > 2 && 2 < nk) issue(std::integral_constant<int, 2>{}, 2);
  if (nk >= D) wait_vm<(D - 1) * NL>();
  else wait_vm<0>();
  step_barrier();
  int ks = 0;
  for (; ks + ST <= nk; ks += ST) {
    step(std::integral_constant<int, 0>{}, ks);
    step(std::integral_constant<int, 1>{}, ks + 1);
    if constexpr (ST > 2) step(std::integral_constant<int, 2>{}, ks + 2);
    if constexpr (ST > 3) step(std::integral_constant<int, 3>{}, ks + 3);
  }
  if (ks < nk) step(std::integral_constant<int, 0>{}, ks);
  if (ks + 1 < nk) step(std::integral_constant<int, 1>{}, ks + 1);
  if constexpr (ST > 2) if (ks + 2 < nk) step(std::integral_constant<int, 2>{}, ks + 2);

  // epilogue: lane holds, for output row m, columns nb .. nb + 3 of each group.  The
  // bias of the wave's columns, and (residual epilogues) the residual of each 32-row
  // group, are loaded before that group's stores: as far as the compiler knows the
  // outputs may alias them, so a load placed after a store would wait on its own,
  // one memory round trip per 4 columns
  typedef typename Elem<T>::vec4 v4;
  typedef typename ResidVec<T, EPI>::type rv_t;
  typedef typename std::conditional<EPI == kEpiResidF32, float, T>::type r_t;
  constexpr bool kRes = EPI == kEpiResidT || EPI == kEpiResidF32;
  v4 bv[NI][4] = {};
  if constexpr (EPI != kEpiPartial) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        bv[i][jj] = *(const v4*)((const T*)g.bias + n0 + wn + 32 * i + 8 * jj + 4 * gq);
  }
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int m = m0 + wm + 32 * j + n;
    rv_t rv[kRes ? NI : 1][4] = {};
    if constexpr (kRes) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (m < g.M)
            rv[i][jj] = *(const rv_t*)((const r_t*)g.resid + (size_t)m * g.ldr + n0 + wn + 32 * i +
                                       8 * jj + 4 * gq);
    }
    if (m >= g.M) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      epilogue_tile<T, EPI>(g, m, n0 + wn + 32 * i, gq, acc[i][j], split, bv[i], rv[kRes ? i : 0]);
  }
}

// LayerNorm gamma and beta of a lane's columns 4 (lane + 64 c) .. + 3, loaded with the
// row (a load placed after the row's first store would wait on its own: the outputs
// may alias gamma and beta as far as the compiler knows).
template <typename T, int NPL>
__device__ __forceinline__ void ln_load_affine(const T* __restrict__ gamma,
                                               const T* __restrict__ beta, int lane,
                                               typename Elem<T>::vec4 gv[NPL],
                                               typename Elem<T>::vec4 bt[NPL]) {
  typedef typename Elem<T>::vec4 v4;
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    gv[c] = *(const v4*)(gamma + 4 * (lane + 64 * c));
    bt[c] = *(const v4*)(beta + 4 * (lane + 64 * c));
  }
}

// (x - mean) * inv * gamma + beta of one row, written as fp32 and / or in T.
template <typename T, int NPL>
__device__ __forceinline__ void ln_write_row(const f32x4 x[NPL], float mean, float inv,
                                             const typename Elem<T>::vec4 gv[NPL],
                                             const typename Elem<T>::vec4 bt[NPL], size_t rowoff,
                                             int lane, float* __restrict__ out_f32,
                                             T* __restrict__ out_t) {
  typedef typename Elem<T>::vec4 v4;
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    const int col = 4 * (lane + 64 * c);
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      y[e] = (x[c][e] - mean) * inv * Elem<T>::to_f(gv[c][e]) + Elem<T>::to_f(bt[c][e]);
    if (out_f32) *(f32x4*)(out_f32 + rowoff + col) = y;
    if (out_t) {
      v4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = Elem<T>::from_f(y[e]);
      *(v4*)(out_t + rowoff + col) = w;
    }
  }
}

// LayerNorm of one row per wave ([FT-LF] steps 5 and 6): mean, biased variance
// (two passes over the row held in registers), (z - mean) / sqrt(var + eps) * gamma
// + beta; written as fp32 (the residual stream) and / or in the layer dtype.
template <typename T, int NPL>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ z,
                                                        const T* __restrict__ gamma,
                                                        const T* __restrict__ beta, float eps,
                                                        int M, int N, float* __restrict__ out_f32,
                                                        T* __restrict__ out_t) {
  typedef typename Elem<T>::vec4 v4;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const float* zr = z + (size_t)row * N;
  f32x4 x[NPL];
#pragma unroll
  for (int c = 0; c < NPL; ++c) x[c] = *(const f32x4*)(zr + 4 * (lane + 64 * c));
  v4 gv[NPL], bt[NPL];
  ln_load_affine<T, NPL>(gamma, beta, lane, gv, bt);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < NPL; ++c) s += (x[c][0] + x[c][1]) + (x[c][2] + x[c][3]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  const float mean = s / (float)N;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < NPL; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dv = x[c][e] - mean;
      q += dv * dv;
    }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) q += __shfl_xor(q, d, 64);
  const float inv = 1.0f / sqrtf(q / (float)N + eps);
  ln_write_row<T, NPL>(x, mean, inv, gv, bt, (size_t)row * N, lane, out_f32, out_t);
}

template <typename T, int TM, int TN, int WAVES, int WM, int WN, int KS, int ST>
hipError_t gemm_launch(const GemmArgs& g, int tiles, hipStream_t st, const GemmArgs* g2 = nullptr) {
  // the second problem's tiles follow the first's (see gemm_kernel)
  const int tiles2 = g2 ? ((g2->M + TM - 1) / TM) * (g2->N / TN) : 0;
  const GemmArgs& h = g2 ? *g2 : g;
  switch (g.epi) {
    case kEpiHeads:
      gemm_kernel<T, kEpiHeads, TM, TN, WAVES, WM, WN, KS, ST><<<tiles + tiles2, 64 * WAVES, 0, st>>>(g, h, tiles);
      break;
    case kEpiGelu:
      gemm_kernel<T, kEpiGelu, TM, TN, WAVES, WM, WN, KS, ST><<<tiles + tiles2, 64 * WAVES, 0, st>>>(g, h, tiles);
      break;
    case kEpiResidT:
      gemm_kernel<T, kEpiResidT, TM, TN, WAVES, WM, WN, KS, ST><<<tiles + tiles2, 64 * WAVES, 0, st>>>(g, h, tiles);
      break;
    case kEpiResidF32:
      gemm_kernel<T, kEpiResidF32, TM, TN, WAVES, WM, WN, KS, ST><<<tiles + tiles2, 64 * WAVES, 0, st>>>(g, h, tiles);
      break;
    case kEpiPartial:
      gemm_kernel<T, kEpiPartial, TM, TN, WAVES, WM, WN, KS, ST><<<tiles + tiles2, 64 * WAVES, 0, st>>>(g, h, tiles);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t gemm_t(const GemmArgs& g, hipStream_t st, const GemmArgs* g2 = nullptr) {
  // 256 x 256 tiles when their grid still covers every CU at least once
  const int big_tiles = g.N % 256 == 0 ? ((g.M + 255) / 256) * (g.N / 256) : 0;
  constexpr int KS = 128 / (int)sizeof(T);   // 128-byte tile rows: 64 fp16 / bf16, 32 fp32
  if (big_tiles >= 256 && g.splits == 1 && (!g2 || g2->N % 256 == 0))
    return gemm_launch<T, 256, 256, 8, 128, 64, KS, 2>(g, big_tiles, st, g2);
  // small grids (at most 320 tiles of 128 x 128, e.g. 1024 rows): 64 x 128 tiles,
  // three workgroups per CU (24 KB of LDS per stage), so more K steps are in flight
  // per CU than with 128 x 128 tiles at two per CU
  const int t128 = ((g.M + 127) / 128) * (g.N / 128) * g.splits;
  if (t128 <= 320)
    return gemm_launch<T, 64, 128, 4, 32, 64, KS, 2>(g, ((g.M + 63) / 64) * (g.N / 128) * g.splits,
                                                     st, g2);
  return gemm_launch<T, 128, 128, 4, 64, 64, KS, 2>(g, t128, st, g2);
}

// LayerNorm of z = sum_s part[s] + bias + resid, one row per wave (the split-K
// reduction of the row's GEMM, in a fixed order, fused into the row kernel).
template <typename T, int NPL, bool RESID_F32>
__global__ __launch_bounds__(256) void layernorm_parts_kernel(
    const float* __restrict__ part, int splits, const T* __restrict__ bias,
    const void* __restrict__ resid, const T* __restrict__ gamma, const T* __restrict__ beta,
    float eps, int M, int N, float* __restrict__ out_f32, T* __restrict__ out_t) {
  typedef typename Elem<T>::vec4 v4;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const size_t sstride = (size_t)M * N;
  const size_t rbase = (size_t)row * N + 4 * lane;   // column chunk c adds 256 c
  // bias and residual first, then the partials GS splits at a time: every load of a
  // group (all column chunks) is issued before its first add.  A group's splits past
  // `splits` read split 0 again and are not added; the sums keep the split order, then
  // add the residual, then the bias.
  constexpr int GS = NPL <= 4 ? 4 : NPL <= 8 ? 2 : 1;
  v4 gv[NPL], bt[NPL];
  ln_load_affine<T, NPL>(gamma, beta, lane, gv, bt);
  f32x4 rv[NPL], bv[NPL];
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    const v4 b4 = *(const v4*)(bias + 4 * lane + 256 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) bv[c][e] = Elem<T>::to_f(b4[e]);
    if (RESID_F32) {
      rv[c] = *(const f32x4*)((const float*)resid + rbase + 256 * c);
    } else {
      const v4 r4 = *(const v4*)((const T*)resid + rbase + 256 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) rv[c][e] = Elem<T>::to_f(r4[e]);
    }
  }
  f32x4 x[NPL];
  for (int s0 = 0; s0 < splits; s0 += GS) {
    f32x4 p[NPL][GS];
#pragma unroll
    for (int c = 0; c < NPL; ++c)
#pragma unroll
      for (int i = 0; i < GS; ++i) {
        const int sp = s0 + i < splits ? s0 + i : 0;
        p[c][i] = *(const f32x4*)(part + sp * sstride + rbase + 256 * c);
      }
#pragma unroll
    for (int c = 0; c < NPL; ++c) {
      if (s0 == 0) x[c] = p[c][0];
      else x[c] += p[c][0];
#pragma unroll
      for (int i = 1; i < GS; ++i)
        if (s0 + i < splits) x[c] += p[c][i];
    }
  }
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    x[c] += rv[c];
    x[c] += bv[c];
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < NPL; ++c) s += (x[c][0] + x[c][1]) + (x[c][2] + x[c][3]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  const float mean = s / (float)N;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < NPL; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dv = x[c][e] - mean;
      q += dv * dv;
    }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) q += __shfl_xor(q, d, 64);
  const float inv = 1.0f / sqrtf(q / (float)N + eps);
  ln_write_row<T, NPL>(x, mean, inv, gv, bt, (size_t)row * N, lane, out_f32, out_t);
}

template <typename T, bool RESID_F32>
hipError_t layernorm_parts_t(const float* part, int splits, const void* bias, const void* resid,
                             const void* gamma, const void* beta, float eps, int M, int N,
                             float* out_f32, void* out_t, hipStream_t st) {
  const int grid = (M + 3) / 4;
  const T* b = (const T*)bias;
  const T* gm = (const T*)gamma;
  const T* bt = (const T*)beta;
  switch (N / 256) {
#define LF_LNP(C)                                                                          \
  case C:                                                                                  \
    layernorm_parts_kernel<T, C, RESID_F32><<<grid, 256, 0, st>>>(part, splits, b, resid, gm, bt, \
                                                                  eps, M, N, out_f32, (T*)out_t); \
    break;
    LF_LNP(1) LF_LNP(2) LF_LNP(3) LF_LNP(4) LF_LNP(8) LF_LNP(16)
#undef LF_LNP
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t layernorm_t(const float* z, const void* gamma, const void* beta, float eps, int M,
                       int N, float* out_f32, void* out_t, hipStream_t st) {
  const int grid = (M + 3) / 4;
  const T* gm = (const T*)gamma;
  const T* bt = (const T*)beta;
  switch (N / 256) {
    case 1: layernorm_kernel<T, 1><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 2: layernorm_kernel<T, 2><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 3: layernorm_kernel<T, 3><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 4: layernorm_kernel<T, 4><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 8: layernorm_kernel<T, 8><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 16: layernorm_kernel<T, 16><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ fused FFN
// [FastFFN] = the page "300%加速！PaddleNLP FastFFN如何让大模型训练"飞"起来", sections
// "FastFFN技术架构" and "技术原理深入解析" (item 1, operator fusion): the FFN's two
// projections and its activation run as one kernel, and the activation is not
// written to global memory.  Here a workgroup owns 32 rows and one slice of the F
// columns.  For each chunk of 32 F columns it forms H = GELU(X W1_c^T + b1_c) in LDS
// (rounded to T, as the two-GEMM path stores its intermediate) and adds H W2_c^T to a
// 32 x D fp32 accumulator held in registers; the accumulator leaves as one fp32
// partial per F slice, and the row LayerNorm kernel sums the partials with b2 and the
// residual ([FT-LF] per-layer step 6).
//
// Wave w: in the first product it takes K range [w D/8, (w + 1) D/8) of the chunk's
// 32 x 32 tile of H^T (the eight K partials are summed in LDS, in a fixed order); in
// the second it owns output columns [w D/8, (w + 1) D/8).  Every W1 and W2 fragment is
// used once per workgroup, so they are read straight into registers: W1 one chunk
// ahead, W2 at the start of its chunk (its latency hides behind the first product).
constexpr int kFfnRows = 32;    // rows per workgroup
constexpr int kFfnChunk = 32;   // F columns per chunk

template <typename T, int NT>   // NT = D / 256: 32-column output tiles per wave
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void ffn_fused_kernel(
    const T* __restrict__ x, const T* __restrict__ w1, const T* __restrict__ b1,
    const T* __restrict__ w2, int M, int F, int f_per_split, float* __restrict__ part) {
  constexpr int D = 256 * NT;
  constexpr int KW = D / 8;             // K columns per wave (first product) = output columns per wave
  constexpr int NK1 = KW / 16;          // MFMAs per wave in the first product
  constexpr int XP = D + 8;             // LDS row pitch of X (elements): rows 16 bytes apart in banks
  constexpr int HP = kFfnChunk + 8;     // LDS row pitch of H
  typedef typename Elem<T>::vec8 v8;
  __shared__ __attribute__((aligned(16))) T xs[kFfnRows * XP];
  __shared__ __attribute__((aligned(16))) float hp[8][16][64];   // K partials of the H^T tile
  __shared__ __attribute__((aligned(16))) T hs[kFfnRows * HP];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const int r0 = blockIdx.x * kFfnRows;
  const int f_lo = blockIdx.y * f_per_split;
  const int nchunk = f_per_split / kFfnChunk;

  // the workgroup's rows of X into LDS (rows past M read zeros)
  const int rows = min(M - r0, kFfnRows);
  const rsrc_t rx = make_rsrc(x + (size_t)r0 * D, (uint32_t)(rows * D * (int)sizeof(T)));
  for (int i = threadIdx.x; i < kFfnRows * D / 8; i += 512) {
    const int r = i / (D / 8), c8 = i % (D / 8);
    *(u32x4*)&xs[r * XP + 8 * c8] =
        __builtin_amdgcn_raw_buffer_load_b128(rx, (r * D + 8 * c8) * (int)sizeof(T), 0, 0);
  }
  const rsrc_t rw1 = make_rsrc(w1, (uint32_t)((size_t)F * D * sizeof(T)));
  const rsrc_t rw2 = make_rsrc(w2, (uint32_t)((size_t)D * F * sizeof(T)));
  // first product: A operand = W1 row f0 + n, k = w KW + 16 i + 8 g (8 elements)
  auto load_w1 = [&](v8 (&f)[NK1], int f0) {
#pragma unroll
    for (int i = 0; i < NK1; ++i)
      f[i] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(
                                        rw1, ((f0 + n) * D + wave * KW + 16 * i + 8 * g) * (int)sizeof(T), 0, 0));
  };
  // second product: A operand = W2 row (output column) w KW + 32 j + n, k = f0 + 16 kk + 8 g
  auto load_w2 = [&](v8 (&f)[NT][2], int f0) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        f[j][kk] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(
                                              rw2, ((wave * KW + 32 * j + n) * F + f0 + 16 * kk + 8 * g) * (int)sizeof(T), 0, 0));
  };

  f32x16 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x16{};
  v8 w1f[NK1];
  load_w1(w1f, f_lo);
  __syncthreads();   // X in LDS
  for (int c = 0; c < nchunk; ++c) {
    const int f0 = f_lo + c * kFfnChunk;
    v8 w2f[NT][2], w1n[NK1];
    load_w2(w2f, f0);
    if (c + 1 < nchunk) load_w1(w1n, f0 + kFfnChunk);
    // H^T tile (F columns f0 .., rows of X) over this wave's K range
    f32x16 h = f32x16{};
#pragma unroll
    for (int i = 0; i < NK1; ++i)
      h = mfma32(w1f[i], *(const v8*)&xs[n * XP + wave * KW + 16 * i + 8 * g], h);
#pragma unroll
    for (int v = 0; v < 16; ++v) hp[wave][v][lane] = h[v];
    __syncthreads();
    // the eight K partials in order, + b1, GELU, rounded to T; element (v, l) of the
    // tile is H[row l % 32][f0 + 8 (v / 4) + 4 (l / 32) + v % 4]
    for (int e = threadIdx.x; e < 16 * 64; e += 512) {
      const int v = e >> 6, l = e & 63;
      float sum = hp[0][v][l];
#pragma unroll
      for (int w = 1; w < 8; ++w) sum += hp[w][v][l];
      const int fi = 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
      sum += Elem<T>::to_f(b1[f0 + fi]);
      hs[(l & 31) * HP + fi] = Elem<T>::from_f(gelu(sum));
    }
    __syncthreads();
    // second product: output columns w KW + 32 j .., rows of X
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const v8 hf = *(const v8*)&hs[n * HP + 16 * kk + 8 * g];
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = mfma32(w2f[j][kk], hf, acc[j]);
    }
    if (c + 1 < nchunk) {
#pragma unroll
      for (int i = 0; i < NK1; ++i) w1f[i] = w1n[i];
    }
  }
  // partial of this F slice: lane holds row r0 + n, columns w KW + 32 j + 8 jj + 4 g .. + 3
  if (r0 + n < M) {
    float* dst = part + ((size_t)blockIdx.y * M + r0 + n) * D + wave * KW + 4 * g;
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *(f32x4*)(dst + 32 * j + 8 * jj) =
            f32x4{acc[j][4 * jj], acc[j][4 * jj + 1], acc[j][4 * jj + 2], acc[j][4 * jj + 3]};
  }
}

template <typename T>
hipError_t ffn_fused_t(const void* x, const void* w1, const void* b1, const void* w2, int M, int D,
                       int F, int splits, float* part, hipStream_t st) {
  const dim3 grid((M + kFfnRows - 1) / kFfnRows, splits);
  const int fps = F / splits;
#define LF_FFN(NT)                                                                          \
  case NT:                                                                                  \
    ffn_fused_kernel<T, NT><<<grid, 512, 0, st>>>((const T*)x, (const T*)w1, (const T*)b1, \
                                                  (const T*)w2, M, F, fps, part);           \
    break;
  switch (D / 256) {
    LF_FFN(1) LF_FFN(2) LF_FFN(3) LF_FFN(4)
    default: return hipErrorInvalidValue;
  }
#undef LF_FFN
  return hipGetLastError();
}

}  // namespace

bool gemm_shape_ok(int M, int N, int K) {
  return M >= 1 && N >= kGT && N % kGT == 0 && K >= kGK && K % kGK == 0;
}

int gemm_splits(int M, int N, int K) {
  const int tiles = ((M + 127) / 128) * (N / 128);
  int s = 1;
  while (s < 16 && tiles * s < 256 && (K / (2 * s)) % 64 == 0 && K / (2 * s) >= 64) s *= 2;
  return s;
}

int ffn_fused_splits(int M, int F) {
  // enough workgroups to fill the chip: split F while there are fewer than 256 row
  // blocks, keeping whole chunks per slice
  const int blocks = (M + kFfnRows - 1) / kFfnRows;
  int s = 1;
  while (s < 16 && blocks * s < 256 && (F / (2 * s)) % kFfnChunk == 0) s *= 2;
  return s;
}

bool ffn_fused_ok(int dtype, int D, int F, int splits) {
  return (dtype == 1 || dtype == 2) && D % 256 == 0 && D >= 256 && D <= 1024 && splits >= 1 &&
         F % (kFfnChunk * splits) == 0 && (int64_t)F * D * 2 <= INT_MAX;
}

hipError_t launch_ffn_fused(int dtype, const void* x, const void* w1, const void* b1,
                            const void* w2, int M, int D, int F, int splits, float* part,
                            hipStream_t st) {
  if (!ffn_fused_ok(dtype, D, F, splits) || M <= 0) return hipErrorInvalidValue;
  if ((int64_t)M * D * 2 > INT_MAX) return hipErrorInvalidValue;
  return dtype == 1 ? ffn_fused_t<f16>(x, w1, b1, w2, M, D, F, splits, part, st)
                    : ffn_fused_t<bf16>(x, w1, b1, w2, M, D, F, splits, part, st);
}

hipError_t launch_layernorm_parts(int dtype, const float* part, int splits, const void* bias,
                                  const void* resid, bool resid_f32, const void* gamma,
                                  const void* beta, float eps, int M, int N, float* out_f32,
                                  void* out_t, hipStream_t st) {
  if (!layernorm_width_ok(N) || splits < 1) return hipErrorInvalidValue;
  switch (dtype) {
    case 0:
      return resid_f32 ? layernorm_parts_t<float, true>(part, splits, bias, resid, gamma, beta,
                                                        eps, M, N, out_f32, out_t, st)
                       : layernorm_parts_t<float, false>(part, splits, bias, resid, gamma, beta,
                                                         eps, M, N, out_f32, out_t, st);
    case 1:
      return resid_f32 ? layernorm_parts_t<f16, true>(part, splits, bias, resid, gamma, beta, eps,
                                                      M, N, out_f32, out_t, st)
                       : layernorm_parts_t<f16, false>(part, splits, bias, resid, gamma, beta, eps,
                                                       M, N, out_f32, out_t, st);
    case 2:
      return resid_f32 ? layernorm_parts_t<bf16, true>(part, splits, bias, resid, gamma, beta,
                                                       eps, M, N, out_f32, out_t, st)
                       : layernorm_parts_t<bf16, false>(part, splits, bias, resid, gamma, beta,
                                                        eps, M, N, out_f32, out_t, st);
  }
  return hipErrorInvalidValue;
}

bool layernorm_width_ok(int N) {
  const int c = N / 256;
  return N % 256 == 0 && (c == 1 || c == 2 || c == 3 || c == 4 || c == 8 || c == 16);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (!gemm_shape_ok(g.M, g.N, g.K)) return hipErrorInvalidValue;
  if (g.splits < 1 || g.K % (64 * g.splits) != 0 || (g.splits > 1) != (g.epi == kEpiPartial))
    return hipErrorInvalidValue;
  switch (g.dtype) {
    case 0: return gemm_t<float>(g, st);
    case 1: return gemm_t<f16>(g, st);
    case 2: return gemm_t<bf16>(g, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_pair(const GemmArgs& g, const GemmArgs& g2, hipStream_t st) {
  if (g.epi != kEpiHeads || g2.epi != kEpiHeads || g.splits != 1 || g2.splits != 1 ||
      g2.dtype != g.dtype || g2.K != g.K)
    return hipErrorInvalidValue;
  if (!gemm_shape_ok(g.M, g.N, g.K) || !gemm_shape_ok(g2.M, g2.N, g2.K)) return hipErrorInvalidValue;
  switch (g.dtype) {
    case 0: return gemm_t<float>(g, st, &g2);
    case 1: return gemm_t<f16>(g, st, &g2);
    case 2: return gemm_t<bf16>(g, st, &g2);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_layernorm(int dtype, const float* z, const void* gamma, const void* beta,
                            float eps, int M, int N, float* out_f32, void* out_t,
                            hipStream_t st) {
  if (!layernorm_width_ok(N)) return hipErrorInvalidValue;
  switch (dtype) {
    case 0: return layernorm_t<float>(z, gamma, beta, eps, M, N, out_f32, out_t, st);
    case 1: return layernorm_t<f16>(z, gamma, beta, eps, M, N, out_f32, out_t, st);
    case 2: return layernorm_t<bf16>(z, gamma, beta, eps, M, N, out_f32, out_t, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lf
