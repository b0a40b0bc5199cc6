// fp16 / bf16 band + global attention on the gfx950 matrix cores, one launch.
//
// [FT-LF] = the page "FasterTransformer Longformer 推理加速实践：PyTorch 集成、输入约束与
// 端到端性能解析", section "Longformer Encoder 计算流程":
//   per-layer step 3  local sliding-window attention plus global attention;
//   per-layer step 4  one masked softmax: a local token normalises over its window
//                     and the global tokens, a global token over the whole
//                     sequence, padded rows are zeroed;
//   preprocessing 1/2 the global-token count and positions, and the local-mask
//                     shift that turns padding into an excluded key.
// The page's design (three window-GEMM segments writing score buffers, a separate
// softmax kernel, a separate global-row pass, preprocessing kernels in front) is
// not followed: scores never leave registers and one launch does everything.  In
// "raw" mode the kernel reads the two masks itself (the count of leading global
// tokens and the live-key test are evaluated where they are used); in "pre" mode
// it reads global_count / the shifted mask produced by the preprocessing entry
// points.
//
// Band workgroup: 4 waves = 128 query rows of one (b, h); wave w owns rows
// r0 + 32w .. r0 + 32w + 31.  Keys move in blocks of 32 rows (K row-major, V
// transposed, plus a per-key 0 / -inf validity term) through a 5-slot LDS ring.
// The key list of a workgroup is
//     [ceil(G/32) global-key blocks][band blocks 0 .. nband+2]
// where band block j holds keys r0 - W/2 + 32j ..; wave w needs band blocks
// w .. w + nband - 1 (nband = (W + 63) / 32).  At step t every wave reads entry t
// (global phase) or t + w (band phase: the waves walk the band on a diagonal, so
// none of them idles); entry t + 4 is written into the ring from registers and the
// loads of entry t + 4 + kDepth are issued (kDepth register sets in flight: memory
// latency is ~1-2 us against ~0.2 us of work per step).  One barrier per step.
//
// Per block and wave: S^T = K Q^T (4 x v_mfma_f32_32x32x16), so each lane holds
// 16 scores of ONE query (lanes n and n + 32 share a query); the running max is
// kept in scaled log2 units and only moved when it grows by more than 8 (then
// p <= 2^8, exact range for fp16 / bf16), so rescaling the accumulators is rare;
// P is rounded to the input type, its row sum is taken from the rounded values
// (v_dot2), then O^T += V^T P^T (4 more MFMAs).
//
// Global rows (r < n_b) attend to all live keys through kg / vg.  The first
// n_split tiles of each (b, h) also take one key split of those rows (split_len
// keys, 32 per wave per round) before their band work: the four wave states are
// merged in LDS and one partial (m, l, o[64]) per row is published with
// agent-scope atomic stores (coherent across XCDs without cache maintenance);
// after them the workgroup takes an atomic ticket, and the one that completes the
// (b, h) reads all partials with agent-scope atomic loads, writes the global rows
// and resets the ticket.
#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32 * kWaves;   // query rows per workgroup
constexpr int kBlk = 32;             // keys per block
constexpr int kKld = 72;             // LDS row pitch of K (elements): 144 B, conflict-free reads
constexpr int kVld = 36;             // LDS row pitch of V^T (elements): 72 B, conflict-free reads
constexpr int kRing = 6;             // LDS block slots
constexpr int kAhead = kWaves + 1;   // entry t + kAhead is written at step t
constexpr int kDepth = 4;            // register sets of loads in flight
constexpr int kStPitch = 67;         // floats per row of a wave state in LDS: m, l, o[64], pad
constexpr int kCombinePairs = 4096;  // (row, split) pairs per combine chunk (2 x 16 KB of LDS)
constexpr int kMaxSplit = 32;        // at most this many key splits per (b, h)
constexpr int kSc1 = 16;             // cache-policy bit of coherent (write-through / bypass) access
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so exp2 never sees inf-inf
constexpr float kLazy = 8.0f;        // move the max only when it grows by more than 2^8

template <typename T>
struct Slot {
  T k[kBlk * kKld];     // K rows of the block
  T vt[64 * kVld];      // V^T: row d holds the 32 keys of the block
  float bias2[kBlk];    // 0 for a live key, -inf for an empty / excluded / padded slot
  int flag;             // 0: every key live, 1: some, 2: none
  int pad[3];
};

static_assert(32 * kStPitch * 4 <= sizeof(Slot<_Float16>), "a wave state fits in one slot");
static_assert(2 * kCombinePairs * 4 <= kRing * sizeof(Slot<_Float16>), "combine buffers fit the ring");

template <typename T>
struct Frag {
  typedef typename Elem<T>::vec8 v8;
  typedef typename Elem<T>::vec4 v4;
  typedef typename Elem<T>::vec2 v2;
};

// ------------------------------------------------------------------ staging
// Loads go through buffer resources sized to one head: a key outside [0, S) is an
// out-of-range offset and reads zeros, so staging has no branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// A key with mask value x is live: raw local mask x == 1, shifted mask x == 0.
template <bool RAW>
__device__ inline bool mask_live(float x) {
  return RAW ? x == 1.0f : x == 0.0f;
}

// Thread t stages K row t/8 (16 B at column 8*(t%8)), V rows 2*(t/16), 2*(t/16)+1
// (8 B each at column 4*(t%16)) and, for t < 32, the mask value of key slot t.
template <typename T>
struct Stage {
  u32x4 k;
  u32x2 v0, v1;
  unsigned short mask_bits;
};

// Block of keys base .. base + 31.  Every thread issues the same four loads (no
// branch), so the compiler can keep later entries in flight while it waits for
// this one.  K / V rows are loaded for every in-range key (a dead key's score is
// masked to -inf, so its data never matters).
template <typename T>
__device__ inline void stage_load(Stage<T>& s, rsrc_t rk, rsrc_t rv, rsrc_t rm, int base) {
  const int t = threadIdx.x;
  const int koff = (t >> 3) * 128 + 16 * (t & 7);
  const int voff = (t >> 4) * 256 + 8 * (t & 15);
  const int b128 = base * 128;
  s.k = __builtin_amdgcn_raw_buffer_load_b128(rk, b128 + koff, 0, 0);
  s.v0 = __builtin_amdgcn_raw_buffer_load_b64(rv, b128 + voff, 0, 0);
  s.v1 = __builtin_amdgcn_raw_buffer_load_b64(rv, b128 + voff + 128, 0, 0);
  s.mask_bits = __builtin_amdgcn_raw_buffer_load_b16(rm, t < kBlk ? 2 * (base + t) : -1, 0, 0);
}

// Write a staged block; key base + j is live iff lo <= key < hi and its mask says so.
template <typename T, bool RAW>
__device__ inline void stage_store(Slot<T>& sl, const Stage<T>& s, int base, int lo, int hi) {
  const int t = threadIdx.x;
  const int kr = t >> 3, kc = t & 7, vp = t >> 4, vc = t & 15;
  *(u32x4*)&sl.k[kr * kKld + 8 * kc] = s.k;
  uint32_t* vt = (uint32_t*)sl.vt;
  constexpr int P = kVld / 2;   // pitch in dwords
  // element i of keys (2vp, 2vp+1) -> V^T[4vc + i][2vp .. 2vp+1] as one dword
  vt[(4 * vc + 0) * P + vp] = (s.v0[0] & 0xffffu) | (s.v1[0] << 16);
  vt[(4 * vc + 1) * P + vp] = (s.v0[0] >> 16) | (s.v1[0] & 0xffff0000u);
  vt[(4 * vc + 2) * P + vp] = (s.v0[1] & 0xffffu) | (s.v1[1] << 16);
  vt[(4 * vc + 3) * P + vp] = (s.v0[1] >> 16) | (s.v1[1] & 0xffff0000u);
  if (wave_id() == 0) {
    const int lane = lane_id();
    const int key = base + lane;
    const bool live = lane < kBlk && key >= lo && key < hi &&
                      mask_live<RAW>(Elem<T>::to_f(__builtin_bit_cast(T, s.mask_bits)));
    const uint64_t bal = __ballot(live);
    if (lane < kBlk) sl.bias2[lane] = live ? 0.0f : -INFINITY;
    if (lane == 0) sl.flag = bal == 0xffffffffull ? 0 : (bal == 0ull ? 2 : 1);
  }
}

// ------------------------------------------------------------------ per-wave math
__device__ inline float cross_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float cross_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
__device__ inline typename Frag<T>::v2 cvt_pair(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 x = {a, b};
  return __builtin_convertvector(x, typename Frag<T>::v2);
}

// Operand fragments of one 32-key block, read from LDS.  K: A operand of
// S^T = K Q^T (lane (n, g) holds key n, dims 16t + 8g ..); V^T: A operand of
// O^T += V^T P^T (lane holds dim 32mb + n, keys 16h + 4g .. +3 and 16h + 8 + 4g ..).
template <typename T>
struct KFrag {
  typename Frag<T>::v8 a[4];
};
template <typename T>
struct VFrag {
  typename Frag<T>::v8 a[2][2];   // [h][mb]
};

template <typename T>
__device__ inline void read_k(KFrag<T>& f, const Slot<T>& sl) {
  typedef typename Frag<T>::v8 v8;
  const int lane = lane_id();
  const int n = lane & 31, g = lane >> 5;
#pragma unroll
  for (int t = 0; t < 4; ++t) f.a[t] = *(const v8*)&sl.k[n * kKld + 16 * t + 8 * g];
}

template <typename T>
__device__ inline void read_v(VFrag<T>& f, const Slot<T>& sl) {
  typedef typename Frag<T>::v4 v4;
  const int lane = lane_id();
  const int n = lane & 31, g = lane >> 5;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const T* row = sl.vt + (32 * mb + n) * kVld + 16 * h + 4 * g;
      const v4 lo = *(const v4*)row;
      const v4 hi = *(const v4*)(row + 8);
      f.a[h][mb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// S^T of one block for the wave's 32 queries (4 MFMAs).
template <typename T>
__device__ inline f32x16 qk_frag(const KFrag<T>& kf, const typename Frag<T>::v8 qf[4]) {
  f32x16 s = f32x16{};
#pragma unroll
  for (int t = 0; t < 4; ++t) s = mfma32(kf.a[t], qf[t], s);
  return s;
}

// O^T += V^T P^T (4 MFMAs).
template <typename T>
__device__ inline void pv_frag(const VFrag<T>& vf, const typename Frag<T>::v8 pf[2], f32x16 o[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) o[mb] = mfma32(vf.a[h][mb], pf[h], o[mb]);
  }
}

// Online-softmax update with the scores s of one block; returns the P^T operand.
// flag (uniform): 0 every key live, else add the per-key 0 / -inf term of `sl`.
// band (uniform): apply |j - s| <= W/2 with c = band_c + 8*(v/4) + (v%4) in 0..W.
// Every block runs the same code on the accumulators (a block without a live key
// adds exact zeros), so the only branch that touches them is the rare rescale.
template <typename T>
__device__ inline void softmax_p(const Slot<T>& sl, const f32x16& s, int flag, f32x16 o[2],
                                 float& m_run, float& l_run, float c2, bool band, int band_c,
                                 int W, typename Frag<T>::v8 pf[2]) {
  typedef typename Frag<T>::v2 v2;
  const int lane = lane_id();
  const int g = lane >> 5;
  float x[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) x[v] = s[v];
  if (flag) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 bb = *(const f32x4*)&sl.bias2[8 * jj + 4 * g];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * jj + i] += bb[i];
    }
  }
  if (band) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = band_c + 8 * (v >> 2) + (v & 3);
      x[v] = (unsigned)c <= (unsigned)W ? x[v] : -INFINITY;
    }
  }
  // max as a tree (short dependency chains)
  float m4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    m4[i] = fmaxf(fmaxf(x[4 * i], x[4 * i + 1]), fmaxf(x[4 * i + 2], x[4 * i + 3]));
  float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
  mx = cross_half_max(mx);
  const float ms = mx * c2;
  const bool need = ms > m_run + kLazy;
  if (__builtin_expect(__ballot(need) != 0ull, 0)) {
    const float m_new = need ? ms : m_run;
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      o[0][v] *= alpha;
      o[1][v] *= alpha;
    }
    m_run = m_new;
  }
  float ls[2] = {0.0f, 0.0f};   // two independent row-sum chains
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = fast_exp2(fmaf(x[8 * h2 + e], c2, -m_run));
      const float p1 = fast_exp2(fmaf(x[8 * h2 + e + 1], c2, -m_run));
      const v2 pp = cvt_pair<T>(p0, p1);
      pf[h2][e] = pp[0];
      pf[h2][e + 1] = pp[1];
      ls[h2] = dot2_ones(pp, ls[h2]);
    }
  }
  l_run += ls[0] + ls[1];
}

// One whole block (used where there is nothing to overlap it with).
template <typename T>
__device__ inline void block_step(const Slot<T>& sl, const typename Frag<T>::v8 qf[4],
                                  f32x16 o[2], float& m_run, float& l_run, float c2, bool band,
                                  int band_c, int W) {
  typedef typename Frag<T>::v8 v8;
  const int flag = __builtin_amdgcn_readfirstlane(sl.flag);
  KFrag<T> kf;
  read_k<T>(kf, sl);
  const f32x16 s = qk_frag<T>(kf, qf);
  VFrag<T> vf;
  read_v<T>(vf, sl);
  v8 pf[2];
  softmax_p<T>(sl, s, flag, o, m_run, l_run, c2, band, band_c, W, pf);
  pv_frag<T>(vf, pf, o);
}

template <typename T>
__device__ inline void load_q(typename Frag<T>::v8 qf[4], const T* __restrict__ rowp, bool ok) {
  typedef typename Frag<T>::v8 v8;
  const int g = lane_id() >> 5;
#pragma unroll
  for (int t = 0; t < 4; ++t) qf[t] = ok ? *(const v8*)(rowp + 16 * t + 8 * g) : v8{};
}

// ------------------------------------------------------------------ workgroup context
template <typename T>
struct Ctx {
  int b, h, bh, tile, S, W, G, nb, ngb, r0, kbase, n_list;
  int n_sp;                  // split entries after the list (4 if this tile carries one)
  int sp_lo, sp_hi;          // key range of the split
  const T *kh, *vh;          // k, v of this head
  const T *kgh, *vgh;        // kg, vg of this head (split tiles; else k, v)
  const T* mask;             // that mask row (raw local mask, or the shifted one)
};

// List entry i: global-key block i (positions 32i.., live below n_b; under the
// head-of-sequence precondition the global positions are 0 .. n_b - 1), band
// block i - ngb (keys kbase + 32(i - ngb).., live in [n_b, S)), or, right after
// the list, the first round of this tile's global-row split (kg / vg keys
// sp_lo + 32(i - n_list).., live in [sp_lo, sp_hi)), which the pipeline thus
// prefetches during the last band steps.  Further entries read out of range (no
// memory traffic) and are never read back.
// (Conditional expressions below pick copied values, never two fields of the
// context: selecting between field addresses would keep the context in memory.)
template <typename T>
__device__ inline int entry_base(const Ctx<T>& c, int i) {
  const int ngb = c.ngb, n_list = c.n_list, S = c.S;
  const int base = i < ngb ? kBlk * i : c.kbase + kBlk * (i - ngb);
  const int sp = c.sp_lo + kBlk * (i - n_list);
  return i < n_list ? base : (i < n_list + c.n_sp ? sp : S);
}

template <typename T>
__device__ inline void load_entry(Stage<T>& s, const Ctx<T>& c, int i) {
  // the choice is uniform: select the (scalar) base pointers, then build the
  // resources, so nothing about the load becomes per-lane
  const bool band = i < c.n_list;
  const uint32_t bytes = (uint32_t)c.S * 128u;
  // select values, not the fields' addresses (keeps the context in registers)
  const T* kp = c.kh;
  const T* vp = c.vh;
  const T* kgp = c.kgh;
  const T* vgp = c.vgh;
  stage_load<T>(s, make_rsrc(band ? kp : kgp, bytes), make_rsrc(band ? vp : vgp, bytes),
                make_rsrc(c.mask, (uint32_t)c.S * 2u), entry_base(c, i));
}

template <typename T, bool RAW>
__device__ inline void store_entry(Slot<T>& sl, const Stage<T>& s, const Ctx<T>& c, int i) {
  const int nb = c.nb, S = c.S, sp_lo = c.sp_lo, sp_hi = c.sp_hi;
  const bool glob = i < c.ngb, band = i < c.n_list;
  const int lo = glob ? 0 : (band ? nb : sp_lo);
  const int hi = glob ? nb : (band ? S : sp_hi);
  stage_store<T, RAW>(sl, s, entry_base(c, i), lo, hi);
}

// ------------------------------------------------------------------ global rows
// Key split `sp` of the global rows of (b, h): partial states into the workspace,
// then the ticket; the workgroup that completes the ticket writes the rows.  The
// first round's four blocks are already in the ring (list entries n_list ..
// n_list + 3); later rounds / query blocks load theirs here.
template <typename T, bool RAW>
__device__ void global_split(const AttnArgs& a, const Ctx<T>& c, int sp, Slot<T>* ring) {
  typedef typename Frag<T>::v8 v8;
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();   // uniform: index math on the scalar unit
  const int n = lane & 31, g = lane >> 5;
  const int G = c.G, nb = c.nb;
  const T* qgh = (const T*)a.qg + (size_t)c.bh * G * 64;
  const int k_lo = c.sp_lo, k_hi = c.sp_hi;
  const int n_rounds = a.split_len / (kBlk * kWaves);
  const float c2 = a.scale * kLog2e;
  float* part = a.partials + ((size_t)c.bh * a.n_split + sp) * (size_t)G * kPartPitch;
  const rsrc_t rpart = make_rsrc(part, (uint32_t)G * kPartPitch * 4u);

  for (int qb = 0; qb * 32 < nb; ++qb) {
    v8 qf[4];
    const int r = 32 * qb + n;
    load_q<T>(qf, qgh + (size_t)(r < nb ? r : 0) * 64, r < nb);
    f32x16 o[2] = {f32x16{}, f32x16{}};
    float m_run = kNegBig, l_run = 0.0f;
    for (int u = 0; u < n_rounds; ++u) {
      int slot = (c.n_list + wave) % kRing;
      if (qb > 0 || u > 0) {
        Stage<T> st[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          stage_load<T>(st[w], make_rsrc(c.kgh, (uint32_t)c.S * 128u),
                        make_rsrc(c.vgh, (uint32_t)c.S * 128u), make_rsrc(c.mask, (uint32_t)c.S * 2u),
                        k_lo + kBlk * (kWaves * u + w));
        __syncthreads();   // earlier readers of the slots are done
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          stage_store<T, RAW>(ring[w], st[w], k_lo + kBlk * (kWaves * u + w), k_lo, k_hi);
        __syncthreads();
        slot = wave;
      }
      block_step<T>(ring[slot], qf, o, m_run, l_run, c2, false, 0, 0);
    }
    __syncthreads();   // every wave is done with its block before the states go in
    float* stp = (float*)&ring[wave];
    const float l_tot = cross_half_sum(l_run);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        stp[n * kStPitch + 2 + 32 * mb + 8 * (v >> 2) + 4 * g + (v & 3)] = o[mb][v];
    if (g == 0) {
      stp[n * kStPitch + 0] = m_run;
      stp[n * kStPitch + 1] = l_tot;
    }
    __syncthreads();
    // merge the four wave states: thread -> (query q, 8 dims); publish with
    // agent-scope atomic stores (write-through, coherent across XCDs)
    {
      const int q = t >> 3, d0 = (t & 7) * 8;
      const int rr = 32 * qb + q;
      float mw[kWaves], M = kNegBig;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = ((const float*)&ring[w])[q * kStPitch];
        M = fmaxf(M, mw[w]);
      }
      float L = 0.0f, acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* sw = (const float*)&ring[w] + q * kStPitch;
        const float f = fast_exp2(mw[w] - M);
        L += sw[1] * f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sw[2 + d0 + i] * f;
      }
      if (rr < nb) {
        // write-through (sc1) stores: visible to every XCD once complete
        const int off = (rr * kPartPitch + 4 + d0) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{acc[0], acc[1], acc[2], acc[3]}),
                                               rpart, off, 0, kSc1);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{acc[4], acc[5], acc[6], acc[7]}),
                                               rpart, off + 16, 0, kSc1);
        if ((t & 7) == 0) {
          const u32x2 ml = {__float_as_uint(M), __float_as_uint(L)};
          __builtin_amdgcn_raw_buffer_store_b64(ml, rpart, rr * kPartPitch * 4, 0, kSc1);
        }
      }
    }
    __syncthreads();   // slots free again
  }

  // ticket: every partial store of this workgroup has completed (write-through)
  // before the ticket is taken
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0) {
    const int old = __hip_atomic_fetch_add(a.counters + c.bh, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == a.n_split - 1;
  }
  __syncthreads();
  if (!s_last) return;
  // merge every split's partial: rows in chunks, (m, l) of all (row, split) pairs
  // into LDS, per-row weights exp2(m - M) / L, then the output dims as weighted
  // sums.  Partials are read with coherent (sc1) loads, all of a thread's loads in
  // flight together; splits past n_split read out of range (zeros, weight 0).
  const int ns = a.n_split;
  const float* pbase = a.partials + (size_t)c.bh * ns * (size_t)G * kPartPitch;
  const rsrc_t rall = make_rsrc(pbase, (uint32_t)ns * G * kPartPitch * 4u);
  const int sstride = G * kPartPitch * 4;   // bytes between splits
  T* outh = (T*)a.out + (size_t)c.b * a.out_sb + (size_t)c.h * a.out_sh;
  float* mw = (float*)ring;                        // [rows][kMaxSplit]: m, then the weight
  float* lw = mw + kCombinePairs;                  // [rows][kMaxSplit]: l
  constexpr int rows_per_chunk = kCombinePairs / kMaxSplit;
  for (int r0 = 0; r0 < nb; r0 += rows_per_chunk) {
    const int nr = min(rows_per_chunk, nb - r0);
    for (int i = t; i < nr * kMaxSplit; i += kThreads) {
      const int rr = r0 + i / kMaxSplit, s2 = i % kMaxSplit;
      const u32x2 ml = __builtin_amdgcn_raw_buffer_load_b64(
          rall, s2 < ns ? s2 * sstride + rr * kPartPitch * 4 : -1, 0, kSc1);
      mw[i] = s2 < ns ? __uint_as_float(ml[0]) : kNegBig;
      lw[i] = __uint_as_float(ml[1]);
    }
    __syncthreads();
    for (int rr = t; rr < nr; rr += kThreads) {
      const float* m_r = mw + rr * kMaxSplit;
      float M = kNegBig;
      for (int s2 = 0; s2 < kMaxSplit; ++s2) M = fmaxf(M, m_r[s2]);
      float L = 0.0f;
      for (int s2 = 0; s2 < kMaxSplit; ++s2) L += lw[rr * kMaxSplit + s2] * fast_exp2(m_r[s2] - M);
      const int pos = RAW ? r0 + rr : a.gidx[(size_t)c.b * c.S + r0 + rr];
      const float inv = mask_live<RAW>(Elem<T>::to_f(c.mask[pos])) ? 1.0f / L : 0.0f;
      for (int s2 = 0; s2 < kMaxSplit; ++s2)
        mw[rr * kMaxSplit + s2] = s2 < ns ? fast_exp2(m_r[s2] - M) * inv : 0.0f;
    }
    __syncthreads();
    for (int idx = t; idx < nr * 16; idx += kThreads) {
      const int rl = idx >> 4, d4 = (idx & 15) * 4;
      const int off0 = ((r0 + rl) * kPartPitch + 4 + d4) * 4;
      f32x4 O = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int h = 0; h < kMaxSplit; h += 16) {
        u32x4 pv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          pv[j] = __builtin_amdgcn_raw_buffer_load_b128(
              rall, h + j < ns ? off0 + (h + j) * sstride : -1, 0, kSc1);
#pragma unroll
        for (int j = 0; j < 16; ++j) O += __builtin_bit_cast(f32x4, pv[j]) * mw[rl * kMaxSplit + h + j];
      }
      typename Frag<T>::v4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = Elem<T>::from_f(O[i]);
      const int pos = RAW ? r0 + rl : a.gidx[(size_t)c.b * c.S + r0 + rl];
      *(typename Frag<T>::v4*)(outh + (size_t)pos * a.out_ss + d4) = w;
    }
    __syncthreads();
  }
  if (t == 0) __hip_atomic_store(a.counters + c.bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ band work
// Entry of wave `wave` at step t: global phase entry t, band phase entry t + wave.
template <typename T>
__device__ inline int wave_entry(const Ctx<T>& c, int t, int wave) {
  return t < c.ngb ? t : t + wave;
}

__device__ inline int xcd_remap(int i, int n) {
  // consecutive workgroup ids go round-robin over the 8 XCDs: give each XCD a
  // contiguous run of logical tiles, so neighbouring tiles of one head share K / V
  // rows in that XCD's L2
  const int per = n / 8;
  const int full = per * 8;
  if (i >= full) return i;
  return (i % 8) * per + i / 8;
}

// Number of global tokens of batch row b: raw mode counts the zeros among the first
// G global-mask values (the tokens are leading, so this is their number); pre mode
// reads global_count.
template <typename T, bool RAW>
__device__ inline int count_globals(const AttnArgs& a, int b) {
  if (!RAW) return min(a.gcnt[b], a.G);
  __shared__ int s_cnt;
  if (threadIdx.x == 0) s_cnt = 0;
  const T* gm = (const T*)a.global_mask + (size_t)b * a.S;
  int cnt = 0;
  for (int s = threadIdx.x; s < a.G; s += kThreads) cnt += Elem<T>::to_f(gm[s]) == 0.0f;
  __syncthreads();
  if (cnt) atomicAdd(&s_cnt, cnt);
  __syncthreads();
  return s_cnt;
}

template <typename T, bool RAW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma_kernel(AttnArgs a, int n_tiles) {
  __shared__ __attribute__((aligned(16))) Slot<T> ring[kRing];
  typedef typename Frag<T>::v8 v8;
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();   // uniform: index math on the scalar unit
  const int n = lane & 31, g = lane >> 5;
  const int n_wg = a.B * a.H * n_tiles;
  // the integer divides below run on the vector ALU; readfirstlane keeps their
  // (uniform) results, and everything derived from them, in scalar registers
  const int li = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, n_wg));

  Ctx<T> c;
  c.bh = __builtin_amdgcn_readfirstlane(li / n_tiles);
  c.tile = __builtin_amdgcn_readfirstlane(li % n_tiles);
  c.b = __builtin_amdgcn_readfirstlane(c.bh / a.H);
  c.h = __builtin_amdgcn_readfirstlane(c.bh % a.H);
  c.S = a.S;
  c.W = a.W;
  c.G = a.G;
  c.ngb = (a.G + kBlk - 1) / kBlk;
  c.r0 = c.tile * kTile;
  c.kbase = c.r0 - (a.W >> 1);
  const int nband = (c.W + 2 * kBlk - 1) / kBlk;
  const int n_steps = c.ngb + nband;
  c.n_list = n_steps + kWaves - 1;
  const size_t head = (size_t)c.bh * c.S * 64;
  c.mask = (const T*)(RAW ? a.local_mask : a.bias) + (size_t)c.b * c.S;
  const float c2 = a.scale * kLog2e;
  const bool split = a.G > 0 && c.tile < a.n_split;
  c.n_sp = split ? kWaves : 0;
  c.sp_lo = split ? c.tile * a.split_len : 0;
  c.sp_hi = split ? min(c.S, c.sp_lo + a.split_len) : 0;
  c.kh = (const T*)a.k + head;
  c.vh = (const T*)a.v + head;
  c.kgh = split ? (const T*)a.kg + head : c.kh;
  c.vgh = split ? (const T*)a.vg + head : c.vh;

  // every load the prologue needs is issued before anything waits
  Stage<T> pro[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) load_entry<T>(pro[i], c, i);
  // Q before the register sets: in the loop its wait count then never holds back
  // the sets in flight
  const int srow = c.r0 + 32 * wave + n;
  v8 qf[4];
  load_q<T>(qf, (const T*)a.q + head + (size_t)(srow < c.S ? srow : 0) * 64, srow < c.S);
  __builtin_amdgcn_sched_barrier(0);
  Stage<T> st[kDepth];   // entry e lives in set e % kDepth
#pragma unroll
  for (int u = 0; u < kDepth; ++u) {
    load_entry<T>(st[(kAhead + u) % kDepth], c, kAhead + u);
    __builtin_amdgcn_sched_barrier(0);
  }
  c.nb = count_globals<T, RAW>(a, c.b);

#pragma unroll
  for (int i = 0; i < kAhead; ++i) store_entry<T, RAW>(ring[i], pro[i], c, i);
  __syncthreads();

  f32x16 o[2] = {f32x16{}, f32x16{}};
  float m_run = kNegBig, l_run = 0.0f;

  // Software pipeline over the wave's blocks: at step t the scores of the next
  // block (entry e(t+1)) go on the matrix cores while the softmax of the current
  // one (entry e(t), scores from the previous step) runs on the vector ALUs, then
  // its PV product is queued.  Entries t .. t+4 are readable at step t; entry t+5
  // is written into the slot entry t-1 used (read for the last time before the
  // previous barrier) and the loads of entry t+5+kDepth are issued into the same
  // register set.  Entries past the list are written and read too (zeros /
  // discarded scores), which keeps the step free of branches around memory
  // operations.  Full groups of kDepth steps run without guards (so the wait
  // counts stay those of the steady state); the remaining steps run once, guarded.
  // step order: every LDS read of the step first (V^T of the current block, K and
  // flag of the next), then the staging, then the softmax on the vector ALUs
  // (hiding the reads' latency), then the next block's QK^T and the current
  // block's PV on the matrix cores, then the barrier.
  f32x16 sc[2];
  int fl[2];   // flag of the block whose scores sit in sc[] (a lane value until used)
  {
    const Slot<T>& s0 = ring[wave_entry(c, 0, wave) % kRing];
    fl[0] = s0.flag;
    KFrag<T> kf;
    read_k<T>(kf, s0);
    sc[0] = qk_frag<T>(kf, qf);
  }
  auto step = [&](int tt, Stage<T>& set, f32x16& s_cur, int& f_cur, f32x16& s_nxt, int& f_nxt) {
    typedef typename Frag<T>::v8 v8;
    const Slot<T>& cs = ring[wave_entry(c, tt, wave) % kRing];
    const Slot<T>& nx = ring[wave_entry(c, tt + 1, wave) % kRing];
    VFrag<T> vf;
    read_v<T>(vf, cs);
    KFrag<T> kf;
    read_k<T>(kf, nx);
    f_nxt = nx.flag;
    __builtin_amdgcn_sched_barrier(0);
    const int e = tt + kAhead;
    store_entry<T, RAW>(ring[e % kRing], set, c, e);
    __builtin_amdgcn_sched_barrier(0);
    load_entry<T>(set, c, e + kDepth);
    __builtin_amdgcn_sched_barrier(0);
    const bool glob = tt < c.ngb;
    const int tb = tt - c.ngb;
    const bool inner = tb >= 1 && kBlk * tb + kBlk - 1 <= c.W;
    v8 pf[2];
    softmax_p<T>(cs, s_cur, __builtin_amdgcn_readfirstlane(f_cur), o, m_run, l_run, c2,
                 !glob && !inner, kBlk * tb + 4 * g - n, c.W, pf);
    s_nxt = qk_frag<T>(kf, qf);
    pv_frag<T>(vf, pf, o);
    __syncthreads();
  };
  static_assert(kDepth % 2 == 0, "score buffers alternate within a group of steps");
  int t0 = 0;
  for (; t0 + kDepth <= n_steps; t0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
      step(t0 + u, st[(u + kAhead) % kDepth], sc[u & 1], fl[u & 1], sc[(u + 1) & 1],
           fl[(u + 1) & 1]);
  }
  // remaining steps, then two drain steps that only write the last two list
  // entries (the split's blocks n_list + 2, n_list + 3, still in registers)
#pragma unroll
  for (int u = 0; u < kDepth + 1; ++u) {
    const int tt = t0 + u;
    if (tt < n_steps) {
      step(tt, st[(u + kAhead) % kDepth], sc[u & 1], fl[u & 1], sc[(u + 1) & 1],
           fl[(u + 1) & 1]);
    } else if (tt < n_steps + 2) {
      const int e = tt + kAhead;
      store_entry<T, RAW>(ring[e % kRing], st[(u + kAhead) % kDepth], c, e);
    }
  }
  __syncthreads();

  // epilogue: normalise and store the local rows
  const float l_tot = cross_half_sum(l_run);
  const bool write = srow < c.S && srow >= c.nb;
  if (write) {
    const bool live = mask_live<RAW>(Elem<T>::to_f(c.mask[srow]));
    const float inv = live ? 1.0f / l_tot : 0.0f;
    T* dst = (T*)a.out + (size_t)c.b * a.out_sb + (size_t)c.h * a.out_sh + (size_t)srow * a.out_ss;
    typedef typename Frag<T>::v4 v4;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        v4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = Elem<T>::from_f(live ? o[mb][4 * jj + i] * inv : 0.0f);
        *(v4*)(dst + 32 * mb + 8 * jj + 4 * g) = w;
      }
    }
  }

  if (split && c.nb > 0) global_split<T, RAW>(a, c, c.tile, ring);
}

template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  const int n_tiles = (a.S + kTile - 1) / kTile;
  const int64_t grid = (int64_t)a.B * a.H * n_tiles;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.G > 0 && (a.split_len % (kBlk * kWaves) != 0 || a.n_split > n_tiles))
    return hipErrorInvalidConfiguration;
  if ((int64_t)a.S * 128 > 0x7fffffff) return hipErrorInvalidValue;   // per-head buffer range
  if (a.ev_begin) {
    hipError_t e0 = hipEventRecord(a.ev_begin, st);
    if (e0 != hipSuccess) return e0;
  }
  if (a.raw)
    attn_mfma_kernel<T, true><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles);
  else
    attn_mfma_kernel<T, false><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_end) e = hipEventRecord(a.ev_end, st);
  return e;
}

}  // namespace

void attn_split_plan(int S, int* n_split, int* split_len) {
  // one split per 128-row tile, at most 32 splits per (b, h); splits are whole
  // rounds of 4 x 32 keys
  const int n_tiles = (S + kTile - 1) / kTile;
  const int want = n_tiles < kMaxSplit ? n_tiles : kMaxSplit;
  const int unit = kBlk * kWaves;
  int len = (S + want - 1) / want;
  len = (len + unit - 1) / unit * unit;
  *split_len = len;
  *n_split = (S + len - 1) / len;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 1: return launch_t<f16>(a, st);
    case 2: return launch_t<bf16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lf
