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
// Band workgroup, two layouts (one per translation unit):
//   8 waves = 256 query rows of one (b, h), two waves per SIMD, an 8-slot LDS ring
//     (146 KB: one workgroup per CU); sequences below 8192 tokens;
//   4 waves = 128 rows, a 4-slot ring (73 KB: two workgroups per CU, one wave of
//     each per SIMD); long sequences, where one workgroup's memory round trips
//     overlap the other's band work.
// Wave w owns the 32 rows r0 + 64 (w % R) + 32 (w / R) .. (R = waves / 2 row groups
// of 64 rows): row group w % R, sub-block w / R.  Keys move in entries of 64 (two
// 32-key blocks; K row-major, V transposed, plus a per-key 0 / -inf term) through the
// ring.  The entry list of a workgroup is
//     [ceil(G/64) global-key entries][band entries 0 .. npb + R - 2]
// where band entry j holds keys r0 - W/2 + 64j ..; row group rg needs band blocks
// 2rg .. 2rg + nband (nband = (W + 63) / 32), i.e. band entries rg .. rg + npb - 1.
// At step t every wave reads entry t (global phase) or t + rg (band phase: the row
// groups walk the band on a diagonal, so none of them idles).  In the helper-wave
// layout (at most 32 global tokens) there is no global phase: the global entry stays
// in the ring's last slot and each sub-block takes its keys in place of a band block
// that lies outside all of its rows' windows (sub-block 1's first, sub-block 0's last),
// the band entries cycling through the other slots.  Entry t + kAhead is
// written into the ring from registers and the loads of entry t + kAhead + 2 are
// issued.  8 waves: kAhead = 5, steps in pairs with one barrier per pair (an entry
// written at step t is first read at step t + 2, after the barrier that ends the pair,
// and the slot it overwrites, entry t - 3's, was last read before the previous
// barrier).  4 waves: kAhead = 2, a barrier after every step (written at t, read from
// t + 1; the slot it overwrites, entry t - 2's, was last read at step t - 2).  Writing
// only a few entries ahead of the read window keeps the workgroups' first loads small,
// so the HBM traffic spreads over the loop instead of arriving as one burst.
//
// Per 32-key block and wave: S^T = K Q^T (4 x v_mfma_f32_32x32x16, accumulator
// initialised with the per-key term, so dead keys cost no vector work), so each
// lane holds 16 scores of ONE query (lanes n and n + 32 share a query).  The
// running max is kept in scaled log2 units, updated once per 64 keys and only moved
// when it grows by more than 8 (then p <= 2^8, exact range for fp16 / bf16), so
// rescaling the accumulators is rare; P is rounded to the input type, its row sum
// is taken from the rounded values (v_dot2), then O^T += V^T P^T (4 more MFMAs).
//
// Global rows (r < n_b) attend to all live keys through kg / vg.  The first
// n_split tiles of each (b, h) also take one key split of those rows (split_len
// keys, 32 per wave per round), after their band work.  The split's first-round
// entries continue the ring's entry list, so the band loop's last steps stage them
// like band entries: their kg / vg loads stream while the loop computes instead of
// joining the launch's first burst of loads.  (4 waves: every other dispatch
// generation runs its split before the band loop instead, so that the two
// workgroups on a CU are in different phases.)  The wave states are merged in LDS
// and one partial (m, l, o[64]) per row is published with write-through stores
// (coherent across XCDs without cache maintenance).  Then the workgroup takes an
// atomic ticket; the one whose ticket completed the (b, h) reads all partials with
// coherent loads, writes the global rows and resets the ticket.
#include <cstdlib>

#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

namespace {

// Two layouts of the band workgroup, one per translation unit (LF_ATTN_WAVES): 8 waves
// = 256 query rows with an 8-slot ring (one workgroup per CU; the default), or 4 waves
// = 128 rows with a 4-slot ring of 75 KB, so that two workgroups share a CU and one's
// memory round trips overlap the other's band work (long sequences).
#ifndef LF_ATTN_WAVES
#define LF_ATTN_WAVES 8
#endif
constexpr int kWaves = LF_ATTN_WAVES;
static_assert(kWaves == 8 || kWaves == 4, "8- or 4-wave layout");
constexpr int kRowGroups = kWaves / 2;   // 64-row groups per workgroup (two sub-blocks each)
constexpr bool kPairs = kWaves == 8;     // one barrier per pair of steps (else per step)
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsW = 32;           // query rows per wave
constexpr int kTile = kRowsW * kWaves;  // query rows per workgroup
constexpr int kBlk = 32;             // keys per MFMA block
constexpr int kEnt = 64;             // keys per ring entry (two blocks)
constexpr int kKld = 72;             // LDS row pitch of K (elements): 144 B, conflict-free reads
constexpr int kVld = 72;             // LDS row pitch of V^T (elements): 144 B, conflict-free reads
constexpr int kRing = kWaves == 8 ? 8 : 4;    // LDS entry slots
constexpr int kAhead = kWaves == 8 ? 5 : 2;   // entry t + kAhead is written at step t
constexpr int kDepth = 2;            // register sets of loads in flight
constexpr int kSplitEnt = kWaves * kBlk / kEnt;   // entries per round of the global-row split
constexpr int kStPitch = 68;         // floats per row of a wave state in LDS: m, l, pad[2], o[64]
constexpr int kMaxSplit = 32;        // at most this many key splits per (b, h)
constexpr int kSc1 = 16;             // cache-policy bit of coherent (write-through / bypass) access
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so exp2 never sees inf-inf
constexpr float kLazy = 8.0f;        // move the max only when it grows by more than 2^8
// Helper waves (8-wave layout): four more waves, one per SIMD, compute the workgroup's
// key split of the global rows while the band waves run the band loop.
constexpr int kHelp = 4;
constexpr int kHelpKeys = 64;        // split keys per helper wave (two 32-key blocks)
constexpr int kHelpSpin = 1 << 22;   // bound of a helper's wait for its predecessor in the merge

template <typename T>
struct Slot {
  T k[kEnt * kKld];     // K rows of the entry
  T vt[64 * kVld];      // V^T: row d holds the 64 keys of the entry
  float bias2[kEnt];    // 0 for a live key, -inf for an empty / excluded / padded slot
};

static_assert(2 * 32 * kStPitch * 4 <= sizeof(Slot<_Float16>), "two wave states fit in one slot");
static_assert(kRing >= kSplitEnt + kWaves / 2, "the split's entries and its wave states fit in the ring");

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

// An entry is staged as 512 parts, kParts per thread: part u = t + kThreads h is
// 16 B of K row u/8 (column 8*(u%8)) and dims 4*(u%16) .. +3 of the key pair
// 2*(u/16), 2*(u/16)+1 of V (8 B each); threads t < 64 also take the mask value of
// key slot t.  Every thread does the same work; no branch.
constexpr int kParts = 512 / kThreads;   // staging parts per thread
template <typename T>
struct Stage {
  u32x4 k[kParts];
  u32x2 v0[kParts], v1[kParts];
  unsigned short mask_bits;
  unsigned short gflag_bits;   // globals-anywhere mode, band entries: global-mask value
};

// Entry of keys base .. base + 63.  Every thread issues the same loads, so the
// compiler can keep later entries in flight while it waits for this one.  K / V
// rows are loaded for every in-range key (a dead key's score is masked to -inf, so
// its data never matters).
template <typename T>
__device__ inline void stage_load(Stage<T>& s, rsrc_t rk, rsrc_t rv, rsrc_t rm, int base) {
  const int t = threadIdx.x;
  const int b128 = base * 128;
#pragma unroll
  for (int h = 0; h < kParts; ++h) {
    const int u = t + kThreads * h;
    const int voff = (u >> 4) * 256 + 8 * (u & 15);
    s.k[h] = __builtin_amdgcn_raw_buffer_load_b128(rk, b128 + (u >> 3) * 128 + 16 * (u & 7), 0, 0);
    s.v0[h] = __builtin_amdgcn_raw_buffer_load_b64(rv, b128 + voff, 0, 0);
    s.v1[h] = __builtin_amdgcn_raw_buffer_load_b64(rv, b128 + voff + 128, 0, 0);
  }
  s.mask_bits = __builtin_amdgcn_raw_buffer_load_b16(rm, t < kEnt ? 2 * (base + t) : -1, 0, 0);
}

// Globals-anywhere mode: global-key entry of slots slot0 .. slot0 + 63, slot r holding
// position gi[r].  Slots below G load (the index holds S positions per row, G <= S);
// slots from n_b on hold ordinary positions and are marked dead when the entry is
// stored (the loads are issued before n_b is known), slots from G on read position
// S, out of range, so their loads return zeros.  Same part mapping as stage_load.
template <typename T>
__device__ inline void stage_gather(Stage<T>& s, rsrc_t rk, rsrc_t rv, rsrc_t rm,
                                   const int32_t* __restrict__ gi, int slot0, int G, int S) {
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < kParts; ++h) {
    const int u = t + kThreads * h;
    const int sk = slot0 + (u >> 3), sv = slot0 + 2 * (u >> 4);
    const int pk = sk < G ? gi[sk] : S;
    const int pv0 = sv < G ? gi[sv] : S;
    const int pv1 = sv + 1 < G ? gi[sv + 1] : S;
    s.k[h] = __builtin_amdgcn_raw_buffer_load_b128(rk, pk * 128 + 16 * (u & 7), 0, 0);
    s.v0[h] = __builtin_amdgcn_raw_buffer_load_b64(rv, pv0 * 128 + 8 * (u & 15), 0, 0);
    s.v1[h] = __builtin_amdgcn_raw_buffer_load_b64(rv, pv1 * 128 + 8 * (u & 15), 0, 0);
  }
  const int sm = slot0 + (t & 63);
  const int pm = sm < G ? gi[sm] : S;
  s.mask_bits = __builtin_amdgcn_raw_buffer_load_b16(rm, t < kEnt ? 2 * pm : -1, 0, 0);
}

// Position of key kk (0..63) inside a V^T row: within each 16-key group, lane group
// g of the PV MFMA needs keys 4g .. 4g+3 and 8+4g .. 8+4g+3 (the row order of the
// score fragment), so those eight are stored together and read as 16 bytes.
__device__ inline int vt_pos(int kk) {
  return (kk & 48) + (kk & 3) + 4 * ((kk >> 3) & 1) + 8 * ((kk >> 2) & 1);
}

// Write a staged entry; key base + j is live iff lo <= key < hi and its mask says so
// (and, with excl_glob, its global-mask value is not zero: a global position is not
// a band key).
template <typename T, bool RAW>
__device__ inline void stage_store(Slot<T>& sl, const Stage<T>& s, int base, int lo, int hi,
                                   bool excl_glob = false) {
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < kParts; ++h) {
    const int u = t + kThreads * h;
    *(u32x4*)&sl.k[(u >> 3) * kKld + 8 * (u & 7)] = s.k[h];
    // dims 4c .. 4c+3 of keys 2vp, 2vp+1 -> V^T rows 4c .. 4c+3, one dword (a key
    // pair) each
    const int vp = u >> 4, cc = u & 15;
    uint32_t* vt = (uint32_t*)sl.vt + vt_pos(2 * vp) / 2;
    constexpr int P = kVld / 2;   // pitch in dwords
    vt[(4 * cc + 0) * P] = __builtin_amdgcn_perm(s.v1[h][0], s.v0[h][0], 0x05040100u);
    vt[(4 * cc + 1) * P] = __builtin_amdgcn_perm(s.v1[h][0], s.v0[h][0], 0x07060302u);
    vt[(4 * cc + 2) * P] = __builtin_amdgcn_perm(s.v1[h][1], s.v0[h][1], 0x05040100u);
    vt[(4 * cc + 3) * P] = __builtin_amdgcn_perm(s.v1[h][1], s.v0[h][1], 0x07060302u);
  }
  if (wave_id() == 0) {
    const int lane = lane_id();
    const int key = base + lane;
    const bool live = key >= lo && key < hi &&
                      mask_live<RAW>(Elem<T>::to_f(__builtin_bit_cast(T, s.mask_bits))) &&
                      !(excl_glob && (s.gflag_bits & 0x7fff) == 0);
    sl.bias2[lane] = live ? 0.0f : -INFINITY;
  }
}

// ------------------------------------------------------------------ per-wave math
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ inline float cross_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// Operand fragments of 32-key block j of an entry, read from LDS.  K: A operand of
// S^T = K Q^T (lane (n, g) holds key 32j + n, dims 16t + 8g ..); V^T: A operand of
// O^T += V^T P^T (lane holds dim 32mb + n, keys 32j + 16h + 4g .. +3 and
// 32j + 16h + 8 + 4g .., stored side by side).
template <typename T>
struct KFrag {
  typename Frag<T>::v8 a[4];
};
template <typename T>
struct VFrag {
  typename Frag<T>::v8 a[2][2];   // [h][mb]
};

template <typename T>
__device__ inline void read_k(KFrag<T>& f, const Slot<T>& sl, int j) {
  typedef typename Frag<T>::v8 v8;
  const int lane = lane_id();
  const int n = lane & 31, g = lane >> 5;
#pragma unroll
  for (int t = 0; t < 4; ++t) f.a[t] = *(const v8*)&sl.k[(kBlk * j + n) * kKld + 16 * t + 8 * g];
}

template <typename T>
__device__ inline void read_v(VFrag<T>& f, const Slot<T>& sl, int j) {
  typedef typename Frag<T>::v8 v8;
  const int lane = lane_id();
  const int n = lane & 31, g = lane >> 5;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      f.a[h][mb] = *(const v8*)(sl.vt + (32 * mb + n) * kVld + kBlk * j + 16 * h + 8 * g);
  }
}

// Per-key term of block j in the accumulator layout (lane (n, g), v -> key
// 32j + 8 (v / 4) + 4 g + v % 4).
template <typename T>
__device__ inline f32x16 read_bias(const Slot<T>& sl, int j) {
  const int g = lane_id() >> 5;
  f32x16 c;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const f32x4 bb = *(const f32x4*)&sl.bias2[kBlk * j + 8 * jj + 4 * g];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[4 * jj + i] = bb[i];
  }
  return c;
}

// S^T of one block plus the per-key term (0 / -inf) as accumulator init: dead keys
// come out at -inf with no vector-ALU work (4 MFMAs).
template <typename T>
__device__ inline f32x16 qk_frag_c(const KFrag<T>& kf, const typename Frag<T>::v8 qf[4],
                                   const f32x16& c) {
  f32x16 s = c;
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

// Row max of 16 scores (NaN-propagating maximum: no operand canonicalisation; the
// scores are never NaN).
__device__ inline float max16(const f32x16& s) {
  float m5[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) m5[i] = vmax(vmax(s[3 * i], s[3 * i + 1]), s[3 * i + 2]);
  const float mx = vmax(vmax(m5[0], m5[1]), vmax(m5[2], s[15]));
  return vmax(vmax(mx, m5[3]), m5[4]);
}

// Band mask of block tq of a sub-block: key kk of the block and query n are within
// the window iff c = 32 tq + kk - n lies in 0 .. W (lane (n, g), v -> kk =
// 8 (v / 4) + 4 g + v % 4).
__device__ inline void band_mask(f32x16& s, int tq, int W) {
  const int lane = lane_id();
  const int band_c = kBlk * tq + 4 * (lane >> 5) - (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int cc = band_c + 8 * (v >> 2) + (v & 3);
    s[v] = (unsigned)cc <= (unsigned)W ? s[v] : -INFINITY;
  }
}

// Rare path: the scaled row max ms grew by more than kLazy over m_run.
__device__ inline void rescale(float ms, f32x16 o[2], float& m_run, float& l_run) {
  const float m_new = ms > m_run + kLazy ? ms : m_run;
  const float alpha = fast_exp2(m_run - m_new);
  l_run *= alpha;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    o[0][v] *= alpha;
    o[1][v] *= alpha;
  }
  m_run = m_new;
}

// P = exp2(c2 s - m), rounded to T, and its row sum.
template <typename T>
__device__ inline void exp_p(const f32x16& s, float m_run, float c2, float& l_run,
                             typename Frag<T>::v8 pf[2]) {
  typedef typename Frag<T>::v2 v2;
  float ls[2] = {0.0f, 0.0f};
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = fast_exp2(fmaf(s[8 * h2 + e], c2, -m_run));
      const float p1 = fast_exp2(fmaf(s[8 * h2 + e + 1], c2, -m_run));
      const v2 pp = cvt_pair<T>(p0, p1);
      pf[h2][e] = pp[0];
      pf[h2][e + 1] = pp[1];
      ls[h2] = dot2_ones(pp, ls[h2]);
    }
  }
  l_run += ls[0] + ls[1];
}

// One whole 32-key block (the global-row split: nothing to overlap it with).
template <typename T>
__device__ inline void block_step(const Slot<T>& sl, int j, const typename Frag<T>::v8 qf[4],
                                  f32x16 o[2], float& m_run, float& l_run, float c2) {
  typedef typename Frag<T>::v8 v8;
  KFrag<T> kf;
  read_k<T>(kf, sl, j);
  const f32x16 s = qk_frag_c<T>(kf, qf, read_bias<T>(sl, j));
  VFrag<T> vf;
  read_v<T>(vf, sl, j);
  const float ms = cross_half_max(max16(s)) * c2;
  if (__builtin_expect(__ballot(ms > m_run + kLazy) != 0ull, 0)) rescale(ms, o, m_run, l_run);
  v8 pf[2];
  exp_p<T>(s, m_run, c2, l_run, pf);
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
  int b, h, bh, tile, S, W, G, nb, ngp, r0, kbase, n_list, npb;
  bool split;                // this tile runs a key split of the global rows
  bool split_tail;           // ... after its band work (its first round staged by the band loop)
  int sp_lo, sp_hi;          // key range of the split
  const T *kh, *vh;          // k, v of this head
  const T *kgh, *vgh;        // kg, vg of this head (split tiles; else k, v)
  const T* mask;             // that mask row (raw local mask, or the shifted one)
  const int32_t* gi;         // globals-anywhere mode: global positions of batch row b
  const unsigned short* gm;  // globals-anywhere mode: global-mask row b (raw bits)
};

// List entry i: global-key entry i (positions 64i.., live below n_b; under the
// head-of-sequence precondition the global positions are 0 .. n_b - 1) or band
// entry i - ngp (keys kbase + 64(i - ngp).., live in [n_b, S)).  Past the list come
// the kSplitEnt entries of the first round of the global-row split (kg / vg keys
// sp_lo + 64(i - n_list).., split tiles only): the band loop's last steps stage them
// like any other entry, so the split after the band work finds them loaded.  Entries
// past those read out of range (no memory traffic) and are never used.
// PAST: entries past the list may be the split's (else they read nothing, and the
// code is shorter).
template <typename T, bool PAST>
__device__ inline int entry_base(const Ctx<T>& c, int i) {
  const int ngp = c.ngp, n_list = c.n_list, S = c.S;
  const int base = i < ngp ? kEnt * i : c.kbase + kEnt * (i - ngp);
  const int e = i - n_list;
  const int past = PAST && c.split_tail && e < kSplitEnt ? c.sp_lo + kEnt * e : S;
  return i < n_list ? base : past;
}

// ANY (globals-anywhere mode): global-key entries gather the global positions
// through the index, band entries also load the global-mask values of their keys.
template <typename T, bool ANY, bool PAST>
__device__ inline void load_entry(Stage<T>& s, const Ctx<T>& c, int i) {
  const uint32_t bytes = (uint32_t)c.S * 128u;
  const bool past = PAST && i >= c.n_list;
  const rsrc_t rk = make_rsrc(past ? c.kgh : c.kh, bytes), rv = make_rsrc(past ? c.vgh : c.vh, bytes);
  const rsrc_t rm = make_rsrc(c.mask, (uint32_t)c.S * 2u);
  if (ANY && i < c.ngp) {
    stage_gather<T>(s, rk, rv, rm, c.gi, kEnt * i, c.G, c.S);
    return;
  }
  const int base = entry_base<T, PAST>(c, i);
  stage_load<T>(s, rk, rv, rm, base);
  if (ANY) {
    const int t = threadIdx.x;
    s.gflag_bits = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(c.gm, (uint32_t)c.S * 2u),
                                                        t < kEnt ? 2 * (base + t) : -1, 0, 0);
  }
}

template <typename T, bool RAW, bool ANY, bool PAST>
__device__ inline void store_entry(Slot<T>& sl, const Stage<T>& s, const Ctx<T>& c, int i) {
  const int nb = c.nb, S = c.S;
  const bool glob = i < c.ngp, past = PAST && i >= c.n_list;
  // band keys: from n_b on when the globals lead, anywhere but the global positions
  // otherwise; split keys: the split's range
  const int lo = past ? c.sp_lo : glob || ANY ? 0 : nb;
  const int hi = past ? c.sp_hi : glob ? nb : S;
  stage_store<T, RAW>(sl, s, entry_base<T, PAST>(c, i), lo, hi, ANY && !glob && !past);
}

// ------------------------------------------------------------------ global rows
// Row q of wave w's state during the split's merge: the slots after the round's
// kSplitEnt entries hold two wave states each.
template <typename T>
__device__ inline float* state_row(Slot<T>* ring, int ebase, int w, int q) {
  unsigned char* sl = (unsigned char*)&ring[(ebase + kSplitEnt + (w >> 1)) % kRing];
  return (float*)(sl + (w & 1) * (32 * kStPitch * 4)) + q * kStPitch;
}

// Key split `sp` of the global rows of (b, h), run after the band work: rounds of
// kWaves blocks (one per wave, four entries), then the wave states are merged in
// LDS and one partial (m, l, o[64]) per row is published with write-through
// stores.  The first round of the first query block is already in the ring (slots
// slot0 .. slot0 + 3, staged by the band loop) and its queries in `qf0` (rows
// 0 .. 31 below G; rows from n_b on are computed but not published).

// ANY is unused in the body: it gives each kernel instantiation a copy of its own
// (with one copy shared by the two raw-mask kernels, the compiler allocated the
// leading-globals kernel's prologue registers worse: 14 spilled VGPRs instead of 1).
// PRE: the first round of the first query block is already in the ring (the band
// loop staged it); else every round loads its entries.
template <typename T, bool RAW, bool ANY, bool PRE>
__device__ void global_split_run(const AttnArgs& a, const Ctx<T>& c, int sp, Slot<T>* ring,
                                 int slot0, const typename Frag<T>::v8 qf0[4]) {
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

  // ring slot of the round's first entry: the staged round sits at slot0, the rounds
  // this function loads at slot 0
  int ebase = PRE ? slot0 : 0;
  for (int qb = 0; qb * 32 < nb; ++qb) {
    v8 qf[4];
    const int r = 32 * qb + n;
    if (qb == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[i] = qf0[i];
    } else {
      load_q<T>(qf, qgh + (size_t)(r < nb ? r : 0) * 64, r < nb);
    }
    f32x16 o[2] = {f32x16{}, f32x16{}};
    float m_run = kNegBig, l_run = 0.0f;
    for (int u = 0; u < n_rounds; ++u) {
      const int base = k_lo + kBlk * kWaves * u;
      const bool staged = PRE && qb == 0 && u == 0;
      if (!staged) {
        ebase = 0;
        Stage<T> st[kSplitEnt];
#pragma unroll
        for (int e = 0; e < kSplitEnt; ++e)
          stage_load<T>(st[e], make_rsrc(c.kgh, (uint32_t)c.S * 128u),
                        make_rsrc(c.vgh, (uint32_t)c.S * 128u), make_rsrc(c.mask, (uint32_t)c.S * 2u),
                        base + kEnt * e);
        __syncthreads();   // earlier readers of the slots are done
#pragma unroll
        for (int e = 0; e < kSplitEnt; ++e)
          stage_store<T, RAW>(ring[e], st[e], base + kEnt * e, k_lo, k_hi);
      }
      __syncthreads();
      block_step<T>(ring[(ebase + (wave >> 1)) % kRing], wave & 1, qf, o, m_run, l_run, c2);
    }
    // the wave states go into the slots the round's entries do not use (two states per
    // slot), so no wave waits for the others before writing its own; only rows below
    // n_b are written and merged
    const int r_valid = min(32, nb - 32 * qb);   // rows of this query block published
    const float l_tot = cross_half_sum(l_run);
    if (n < r_valid) {
      float* stp = state_row(ring, ebase, wave, n);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *(f32x4*)&stp[4 + 32 * mb + 8 * jj + 4 * g] =
              f32x4{o[mb][4 * jj], o[mb][4 * jj + 1], o[mb][4 * jj + 2], o[mb][4 * jj + 3]};
      if (g == 0) {
        stp[0] = m_run;
        stp[1] = l_tot;
      }
    }
    __syncthreads();
    // merge the wave states: thread -> (query q, 8 dims) (threads from 256 on idle);
    // publish with write-through stores (coherent across XCDs)
    constexpr int kTpr = 8, kDpt = 64 / kTpr;   // threads per row, dims each
    const int q = t / kTpr, d0 = (t % kTpr) * kDpt;
    if (q < r_valid) {
      float mw[kWaves], M = kNegBig;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = state_row(ring, ebase, w, q)[0];
        M = fmaxf(M, mw[w]);
      }
      float L = 0.0f;
      f32x4 acc[kDpt / 4];
#pragma unroll
      for (int i = 0; i < kDpt / 4; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* sw = state_row(ring, ebase, w, q);
        const float f = fast_exp2(mw[w] - M);
        L += sw[1] * f;
#pragma unroll
        for (int i = 0; i < kDpt / 4; ++i) acc[i] += *(const f32x4*)&sw[4 + d0 + 4 * i] * f;
      }
      const int rr = 32 * qb + q;
      const int off = (rr * kPartPitch + 4 + d0) * 4;
#pragma unroll
      for (int i = 0; i < kDpt / 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i]), rpart, off + 16 * i,
                                               0, kSc1);
      if (d0 == 0) {
        const u32x2 ml = {__float_as_uint(M), __float_as_uint(L)};
        __builtin_amdgcn_raw_buffer_store_b64(ml, rpart, rr * kPartPitch * 4, 0, kSc1);
      }
    }
    __syncthreads();   // slots free again
  }
}

// Ticket of a split workgroup, taken right after its partial is published: every
// wave waits for its write-through stores, then one atomic increment (its old value,
// in thread 0, tells whether this workgroup's partial completed the (b, h)).
template <typename T>
__device__ inline int take_ticket(const AttnArgs& a, const Ctx<T>& c) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int old = 0;
  if (threadIdx.x == 0)
    old = __hip_atomic_fetch_add(a.counters + c.bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

// Run by the workgroup whose ticket completed the (b, h): merges every split's
// partial and writes the global rows, thread per (row, 4 dims); the (m, l) and o of
// 16 splits per round are loaded together with coherent (sc1) loads, splits past
// n_split read out of range and get weight 0.
template <typename T, bool RAW, bool ANY>
__device__ void global_combine(const AttnArgs& a, const Ctx<T>& c) {
  const int t = threadIdx.x;
  const int G = c.G, nb = c.nb, ns = a.n_split;
  const float* pbase = a.partials + (size_t)c.bh * ns * (size_t)G * kPartPitch;
  const rsrc_t rall = make_rsrc(pbase, (uint32_t)ns * G * kPartPitch * 4u);
  const int sstride = G * kPartPitch * 4;   // bytes between splits
  T* outh = (T*)a.out + (size_t)c.b * a.out_sb + (size_t)c.h * a.out_sh;
  for (int idx = t; idx < nb * 16; idx += kThreads) {
    const int rl = idx >> 4, d4 = (idx & 15) * 4;
    // the row's position and mask value first: their loads travel with the partials'
    const int pos = RAW && !ANY ? rl : a.gidx[(size_t)c.b * c.S + rl];
    const T mval = c.mask[pos];
    const int off_ml = rl * kPartPitch * 4, off_o = (rl * kPartPitch + 4 + d4) * 4;
    float M = kNegBig, L = 0.0f;
    f32x4 O = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int h = 0; h < ns; h += 16) {
      u32x2 ml[16];
      u32x4 pv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool ok = h + j < ns;
        ml[j] = __builtin_amdgcn_raw_buffer_load_b64(rall, ok ? (h + j) * sstride + off_ml : -1, 0, kSc1);
        pv[j] = __builtin_amdgcn_raw_buffer_load_b128(rall, ok ? (h + j) * sstride + off_o : -1, 0, kSc1);
      }
      float m[16];
      float mh = M;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        m[j] = h + j < ns ? __uint_as_float(ml[j][0]) : kNegBig;
        mh = fmaxf(mh, m[j]);
      }
      const float sc = fast_exp2(M - mh);
      L *= sc;
      O *= sc;
      M = mh;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float w = h + j < ns ? fast_exp2(m[j] - M) : 0.0f;
        L += __uint_as_float(ml[j][1]) * w;
        O += __builtin_bit_cast(f32x4, pv[j]) * w;
      }
    }
    const float inv = mask_live<RAW>(Elem<T>::to_f(mval)) ? 1.0f / L : 0.0f;
    typename Frag<T>::v4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = Elem<T>::from_f(O[i] * inv);
    *(typename Frag<T>::v4*)(outh + (size_t)pos * a.out_ss + d4) = w;
  }
  __syncthreads();
  if (t == 0) __hip_atomic_store(a.counters + c.bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ band work
// Entry of row group rg at step t: global phase entry t, band phase entry t + rg
// (row group rg's first band block is 2rg: its 64 rows start 64 rg after the
// tile's).
template <typename T>
__device__ inline int wave_entry(const Ctx<T>& c, int t, int rg) {
  return t < c.ngp ? t : t + rg;
}

// Ring slot of list entry i.  FOLD (the helper-wave layout, exactly one global-key
// entry): the global entry stays in the last slot for the whole loop and the band
// entries cycle through the other kRing - 1.  Seven slots suffice for the band: in
// the pair of steps (t, t + 1) entries t .. t + 4 are read and t + 5, t + 6 are
// written, which take the slots of entries t - 2 and t - 1, both last read before
// the barrier that ended the previous pair.
template <bool FOLD>
__device__ inline int ring_slot(int i) {
  return FOLD ? (i == 0 ? kRing - 1 : (i - 1) % (kRing - 1)) : i % kRing;
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

// Number of global tokens of batch row b: raw mode counts the zeros (+0 or -0: the
// bits other than the sign are clear, in fp16 and bf16 alike) among the first G
// global-mask values (the tokens are leading, so this is their number); pre mode and
// the globals-anywhere mode read global_count.  Wave 0 counts with ballots (count_load
// issues the first load of the workgroup, the first 64 mask values, one per lane; since
// vector loads complete in order, the wait in count_globals does not wait for the
// staging loads issued after it).
template <typename T, bool RAW, bool ANY>
__device__ inline int count_load(const AttnArgs& a, int b) {
  if (!RAW || ANY) return a.gcnt[b];
  const unsigned short* gm = (const unsigned short*)a.global_mask + (size_t)b * a.S;
  const int lane = lane_id();
  return lane < a.G ? gm[lane] : 0x3c00;   // 0x3c00: not a zero
}

template <typename T, bool RAW, bool ANY>
__device__ inline int count_globals(const AttnArgs& a, int b, int first) {
  if (!RAW || ANY) return min(first, a.G);
  const unsigned short* gm = (const unsigned short*)a.global_mask + (size_t)b * a.S;
  int cnt = __builtin_popcountll(__ballot((first & 0x7fff) == 0));
  for (int s0 = 64; s0 < a.G; s0 += 64) {
    const int s = s0 + lane_id();
    const int x = s < a.G ? gm[s] : 0x3c00;
    cnt += __builtin_popcountll(__ballot((x & 0x7fff) == 0));
  }
  return __builtin_amdgcn_readfirstlane(cnt);
}

// Global rows of one (b, h) in a workgroup of their own (GWG mode, used when the
// band tiles leave CUs idle): one split over every key, its partial merged by the
// same workgroup; it runs beside the band tiles, which then skip the split, the
// ticket and the combine.
template <typename T, bool RAW, bool ANY>
__device__ void global_rows_wg(const AttnArgs& a, Slot<T>* ring, int bh) {
  typedef typename Frag<T>::v8 v8;
  Ctx<T> c;
  c.bh = bh;
  c.b = __builtin_amdgcn_readfirstlane(bh / a.H);
  c.h = __builtin_amdgcn_readfirstlane(bh % a.H);
  c.S = a.S;
  c.W = a.W;
  c.G = a.G;
  c.ngp = (a.G + kEnt - 1) / kEnt;
  c.tile = 0;
  c.r0 = 0;
  c.kbase = 0;
  c.n_list = 0;
  c.mask = (const T*)(RAW ? a.local_mask : a.bias) + (size_t)c.b * c.S;
  c.gi = ANY ? a.gidx + (size_t)c.b * c.S : nullptr;
  c.gm = ANY ? (const unsigned short*)a.global_mask + (size_t)c.b * c.S : nullptr;
  c.split = true;
  c.sp_lo = 0;
  c.sp_hi = c.S;
  const size_t head = (size_t)bh * c.S * 64;
  c.kh = (const T*)a.k + head;
  c.vh = (const T*)a.v + head;
  c.kgh = (const T*)a.kg + head;
  c.vgh = (const T*)a.vg + head;
  const int first = count_load<T, RAW, ANY>(a, c.b);
  c.nb = count_globals<T, RAW, ANY>(a, c.b, first);
  if (c.nb == 0) return;
  const int n = lane_id() & 31;
  v8 qg0[4];
  load_q<T>(qg0, (const T*)a.qg + ((size_t)bh * a.G + (n < a.G ? n : 0)) * 64, n < a.G);
  global_split_run<T, RAW, ANY, false>(a, c, 0, ring, 0, qg0);
  __builtin_amdgcn_s_waitcnt(0);   // the partial's write-through stores are complete
  __syncthreads();
  global_combine<T, RAW, ANY>(a, c);
}

// ------------------------------------------------------------------ helper waves
constexpr int kMergeRows = 16;   // query rows per pass of the helpers' merge
// LDS of the helper waves: the states of helpers 0 .. 2 for one pass of the merge
// (layout of a wave state: m, l, pad, pad, o[64] per row), the merge's counters and
// the ticket's outcome.
struct HelpLds {
  float st[kHelp - 1][kMergeRows * kStPitch];
  int written;   // states written by helpers 0 .. 2, over all passes
  int read;      // passes helper 3 has read
  int last;      // this workgroup's ticket completed the (b, h)
};

// Rows of the global-row combine (every split's partial merged, the global rows
// written), lanes t0, t0 + stride, .. of the calling threads: thread per (row, 4
// dims); the (m, l) and o of 16 splits per round are loaded together with coherent
// (sc1) loads.  No barrier: used by one helper wave.
template <typename T, bool RAW, bool ANY>
__device__ void combine_rows(const AttnArgs& a, const Ctx<T>& c, int t0, int stride) {
  const int G = c.G, nb = c.nb, ns = a.n_split;
  const float* pbase = a.partials + (size_t)c.bh * ns * (size_t)G * kPartPitch;
  const rsrc_t rall = make_rsrc(pbase, (uint32_t)ns * G * kPartPitch * 4u);
  const int sstride = G * kPartPitch * 4;   // bytes between splits
  T* outh = (T*)a.out + (size_t)c.b * a.out_sb + (size_t)c.h * a.out_sh;
  for (int idx = t0; idx < nb * 16; idx += stride) {
    const int rl = idx >> 4, d4 = (idx & 15) * 4;
    const int pos = RAW && !ANY ? rl : a.gidx[(size_t)c.b * c.S + rl];
    const T mval = c.mask[pos];
    const int off_ml = rl * kPartPitch * 4, off_o = (rl * kPartPitch + 4 + d4) * 4;
    float M = kNegBig, L = 0.0f;
    f32x4 O = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int h = 0; h < ns; h += 16) {
      u32x2 ml[16];
      u32x4 pv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool ok = h + j < ns;
        ml[j] = __builtin_amdgcn_raw_buffer_load_b64(rall, ok ? (h + j) * sstride + off_ml : -1, 0, kSc1);
        pv[j] = __builtin_amdgcn_raw_buffer_load_b128(rall, ok ? (h + j) * sstride + off_o : -1, 0, kSc1);
      }
      float m[16];
      float mh = M;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        m[j] = h + j < ns ? __uint_as_float(ml[j][0]) : kNegBig;
        mh = fmaxf(mh, m[j]);
      }
      const float sc = fast_exp2(M - mh);
      L *= sc;
      O *= sc;
      M = mh;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float w = h + j < ns ? fast_exp2(m[j] - M) : 0.0f;
        L += __uint_as_float(ml[j][1]) * w;
        O += __builtin_bit_cast(f32x4, pv[j]) * w;
      }
    }
    const float inv = mask_live<RAW>(Elem<T>::to_f(mval)) ? 1.0f / L : 0.0f;
    typename Frag<T>::v4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = Elem<T>::from_f(O[i] * inv);
    *(typename Frag<T>::v4*)(outh + (size_t)pos * a.out_ss + d4) = w;
  }
}

// Bounded wait of a helper wave until an LDS counter reaches `target` (every wave of
// the workgroup is resident and the waits form no cycle, so it always ends).
__device__ inline void help_wait(const int* ctr, int target) {
  for (int it = 0; it < kHelpSpin; ++it) {
    if (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Helper wave hw (0 .. 3) of a band workgroup whose tile takes a key split of the
// global rows (n_b <= 32 rows, one query block): keys sp_lo + 64 hw .. + 63 of kg / vg.
// Its work is cut into phases between the barriers the band waves execute (n_bar of
// them in all), so that no band wave waits for it:
//   loads (with four or more barriers they are issued after the first one and with
//   five or more K and V go out one pair of steps apart, so they do not join the
//   launch's first burst of loads; the combine then runs after the band waves' last
//   barrier, beside their last step and epilogue);
//   work phase: S^T = K Q^T with the per-key term as accumulator init, the exact row
//     max over its 64 keys, P rounded to T, O^T = V^T P^T, V^T formed on the matrix
//     core from row-major V; helpers 0 .. 2 write their states to LDS and helper 3
//     merges the four in a fixed order (so the result does not depend on timing) and
//     publishes the partial with write-through stores, 16 rows per pass;
//   ticket phase: helper 3 waits for its stores and takes the (b, h) ticket;
//   combine phase: the helpers of the workgroup whose ticket completed the (b, h)
//     merge all partials and write the global rows;
// then the remaining barriers.
template <typename T, bool RAW, bool ANY>
__device__ void help_run(const AttnArgs& a, const Ctx<T>& c0, int n_bar, HelpLds& hl,
                         const int* s_nb) {
  typedef typename Frag<T>::v8 v8;
  // the helper's work is short and sits on the band waves' barrier schedule: issue
  // before the (older) band waves of the SIMD when both are ready
  __builtin_amdgcn_s_setprio(2);
  const int hw = wave_id() - kWaves;
  const int lane = lane_id();
  const int n = lane & 31, g = lane >> 5;
  Ctx<T> c = c0;
  const bool split = a.G > 0 && c.tile < a.n_split;
  const int sp = c.tile;
  const int k0 = sp * a.split_len + kHelpKeys * hw;   // first key of this helper
  const int k_hi = min(c.S, sp * a.split_len + a.split_len);
  const float c2 = a.scale * kLog2e;
  const size_t head = (size_t)c.bh * c.S * 64;
  const uint32_t bytes = (uint32_t)c.S * 128u;
  const rsrc_t rk = make_rsrc((const T*)a.kg + head, bytes);
  const rsrc_t rv = make_rsrc((const T*)a.vg + head, bytes);
  const rsrc_t rm = make_rsrc(c.mask, (uint32_t)c.S * 2u);
  // with barriers to spare, the loads go out after the band waves' first burst of
  // loads, K in the band loop's first pair of steps and V in the second, so that their
  // 64 KB per workgroup spread over the loop's own traffic
  const int n_wait = n_bar >= 5 ? 2 : n_bar >= 4 ? 1 : 0;
  // K and V rows in the A-operand layout (lane (n, g): key 32 j + n, dims 16 t + 8 g ..),
  // 16-byte loads
  v8 qf[4];
  v8 kf[2][4], vr[2][4];
  unsigned short mbits = 0;
  auto issue_k = [&]() {   // the queries, K rows and the keys' mask values
    load_q<T>(qf, (const T*)a.qg + ((size_t)c.bh * a.G + (n < a.G ? n : 0)) * 64, n < a.G);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int off = (k0 + 32 * j + n) * 128 + 2 * (16 * t + 8 * g);
        kf[j][t] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      }
    mbits = __builtin_amdgcn_raw_buffer_load_b16(rm, 2 * (k0 + lane), 0, 0);
  };
  auto issue_v = [&]() {   // the V rows
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int off = (k0 + 32 * j + n) * 128 + 2 * (16 * t + 8 * g);
        vr[j][t] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
      }
  };
  if (split && n_wait == 0) {
    issue_k();
    issue_v();
  }
  if (hw == 0 && lane == 0) {
    hl.written = 0;
    hl.read = 0;
  }
  __syncthreads();   // barrier 0: the band prologue's
  c.nb = __builtin_amdgcn_readfirstlane(*s_nb);
  if (n_wait) {
    if (split) {
      issue_k();
      if (n_wait == 1) issue_v();
    }
    __syncthreads();   // barrier 1
    if (n_wait == 2) {
      if (split) issue_v();
      __syncthreads();   // barrier 2
    }
  }
  const bool work = split && c.nb > 0;
  if (work) {
    // per-key term: live key of the split range with a live mask value
    const bool live = k0 + lane < k_hi && mask_live<RAW>(Elem<T>::to_f(__builtin_bit_cast(T, mbits)));
    const uint64_t lv = __ballot(live);
    f32x16 sc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = 32 * j + 8 * (v >> 2) + 4 * g + (v & 3);
        sc[j][v] = (lv >> kk) & 1 ? 0.0f : -INFINITY;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) sc[j] = mfma32(kf[j][t], qf[t], sc[j]);
    }
    // V^T fragments from the row-major V on the matrix core: D = V_rows x E, where the
    // B operand E places dims 16 t' .. 16 t' + 15 at columns 16 t' (exact: every
    // product is x * 1 or x * 0), leaves lane (n, g) holding dim 32 mb + n of keys
    // 8 (v / 4) + 4 g + v % 4 of the block, which is the PV operand's key order
    v8 e_lo, e_hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      e_lo[e] = Elem<T>::from_f(n == 8 * g + e ? 1.0f : 0.0f);
      e_hi[e] = Elem<T>::from_f(n == 16 + 8 * g + e ? 1.0f : 0.0f);
    }
    const float m_h = fmaxf(cross_half_max(vmax(max16(sc[0]), max16(sc[1]))) * c2, kNegBig);
    float l_h = 0.0f;
    f32x16 o[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      VFrag<T> vv;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 d = mfma32(vr[j][2 * mb], e_lo, f32x16{});
        d = mfma32(vr[j][2 * mb + 1], e_hi, d);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const typename Frag<T>::v2 pp = cvt_pair<T>(d[8 * h + e], d[8 * h + e + 1]);
            vv.a[h][mb][e] = pp[0];
            vv.a[h][mb][e + 1] = pp[1];
          }
      }
      v8 pf[2];
      exp_p<T>(sc[j], m_h, c2, l_h, pf);
      pv_frag<T>(vv, pf, o);
    }
    l_h = cross_half_sum(l_h);
    // merge: 16 query rows per pass; helpers 0 .. 2 write their states, helper 3 merges
    // them with its own in the order 0, 1, 2, 3 and publishes
    const int r_valid = min(32, c.nb);
    float* part = a.partials + ((size_t)c.bh * a.n_split + sp) * (size_t)c.G * kPartPitch;
    const rsrc_t rpart = make_rsrc(part, (uint32_t)c.G * kPartPitch * 4u);
    const int n_pass = (r_valid + kMergeRows - 1) / kMergeRows;
    for (int ps = 0; ps < n_pass; ++ps) {
      const int r = n - kMergeRows * ps;
      const bool mine = r >= 0 && r < kMergeRows && n < r_valid;
      if (hw < kHelp - 1) {
        if (ps > 0) help_wait(&hl.read, ps);   // helper 3 has read the previous pass
        if (mine) {
          float* row = hl.st[hw] + r * kStPitch;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              *(f32x4*)&row[4 + 32 * mb + 8 * jj + 4 * g] =
                  f32x4{o[mb][4 * jj], o[mb][4 * jj + 1], o[mb][4 * jj + 2], o[mb][4 * jj + 3]};
          if (g == 0) {
            row[0] = m_h;
            row[1] = l_h;
          }
        }
        // one count per wave (the release orders every lane's writes before it)
        if (lane == 0) __hip_atomic_fetch_add(&hl.written, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        help_wait(&hl.written, (kHelp - 1) * (ps + 1));
        if (mine) {
          float mw[kHelp], M = m_h;
#pragma unroll
          for (int w = 0; w < kHelp - 1; ++w) {
            mw[w] = hl.st[w][r * kStPitch];
            M = fmaxf(M, mw[w]);
          }
          mw[kHelp - 1] = m_h;
          float wt[kHelp], L = 0.0f;
#pragma unroll
          for (int w = 0; w < kHelp; ++w) {
            wt[w] = fast_exp2(mw[w] - M);
            L += (w < kHelp - 1 ? hl.st[w][r * kStPitch + 1] : l_h) * wt[w];
          }
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int d = 4 + 32 * mb + 8 * jj + 4 * g;
              f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
              for (int w = 0; w < kHelp - 1; ++w) acc += *(const f32x4*)&hl.st[w][r * kStPitch + d] * wt[w];
              acc += f32x4{o[mb][4 * jj], o[mb][4 * jj + 1], o[mb][4 * jj + 2], o[mb][4 * jj + 3]} *
                     wt[kHelp - 1];
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), rpart,
                                                     (n * kPartPitch + d) * 4, 0, kSc1);
            }
          if (g == 0) {
            const u32x2 ml = {__float_as_uint(M), __float_as_uint(L)};
            __builtin_amdgcn_raw_buffer_store_b64(ml, rpart, n * kPartPitch * 4, 0, kSc1);
          }
        }
        __hip_atomic_store(&hl.read, ps + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
  __syncthreads();   // barrier 1 + n_wait
  if (work && hw == kHelp - 1) {
    __builtin_amdgcn_s_waitcnt(0);   // the partial's write-through stores are complete
    if (lane == 0) {
      const int old = __hip_atomic_fetch_add(a.counters + c.bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // every split has published: the ticket is ready for the next launch
      if (old == a.n_split - 1)
        __hip_atomic_store(a.counters + c.bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      hl.last = old == a.n_split - 1;
    }
  }
  __syncthreads();   // barrier 2 + n_wait
  // the four helpers of the workgroup that completed the (b, h) write its global rows
  if (work && hl.last) combine_rows<T, RAW, ANY>(a, c, 64 * hw + lane, 64 * kHelp);
  for (int i = 3 + n_wait; i < n_bar; ++i) __syncthreads();
}

// One step t of a wave: the two 32-key blocks of its entry.  LDS reads first
// (K, V^T and per-key terms of both blocks), then QK^T, the band mask on edge
// steps only, one running-max update for the 64 keys, P, PV, then the staging of
// entry t + kAhead and the loads of entry t + kAhead + kDepth, then (BAR: second
// step of a pair) the barrier.  Entries t .. t + 3 are read during the step and
// t + 5 is written.
// LATE_V (the helper-wave layout, 168 registers per wave): the V^T fragments are read
// after the QK^T MFMAs are issued, into the registers the K fragments leave, and
// arrive while the max and P are computed.
// FOLD (the helper-wave layout): sub-block 1's first band block (tq = -1) and
// sub-block 0's last one (tq = 2 npb - 1 >= nband) lie wholly outside the window of
// every row of the sub-block; in their place the wave takes the global keys (block 0
// of the global entry, which holds them all when there are at most 32), so no step of
// the loop is spent on the global keys alone (sub-block 1 substitutes block 0 at the
// first band step, sub-block 0 block 1 at the last; wave-uniform scalar selects of the
// LDS base).  The global keys' scores then join the running max one step apart in the
// two sub-blocks instead of first: the same sums in another order.
template <typename T, bool RAW, bool ANY, bool PAST, bool BAR, bool LATE_V, bool FOLD>
__device__ __forceinline__ void band_step(const Ctx<T>& c, Slot<T>* ring, int tt, int rg, int sb,
                                          float c2, Stage<T>& set,
                                          const typename Frag<T>::v8 qf[4], f32x16 o[2],
                                          float& m_run, float& l_run) {
  typedef typename Frag<T>::v8 v8;
  const Slot<T>& cs = ring[ring_slot<FOLD>(wave_entry(c, tt, rg))];
  const int bt = tt - c.ngp;
  const bool gs0 = FOLD && sb == 1 && bt == 0;
  const bool gs1 = FOLD && sb == 0 && bt == c.npb - 1;
  const Slot<T>& cs0 = gs0 ? ring[kRing - 1] : cs;
  const Slot<T>& cs1 = gs1 ? ring[kRing - 1] : cs;
  const int j1 = gs1 ? 0 : 1;
  KFrag<T> kf0, kf1;
  read_k<T>(kf0, cs0, 0);
  read_k<T>(kf1, cs1, j1);
  const f32x16 c0 = read_bias<T>(cs0, 0), c1 = read_bias<T>(cs1, j1);
  VFrag<T> vf0, vf1;
  if (!LATE_V) {
    read_v<T>(vf0, cs0, 0);
    read_v<T>(vf1, cs1, j1);
  }
  f32x16 s0 = qk_frag_c<T>(kf0, qf, c0);
  f32x16 s1 = qk_frag_c<T>(kf1, qf, c1);
  if (LATE_V) {
    __builtin_amdgcn_sched_barrier(0);
    read_v<T>(vf0, cs0, 0);
    read_v<T>(vf1, cs1, j1);
  }
  // blocks tq = 1 .. (W - 31) / 32 of a sub-block lie wholly inside the window of
  // every row; the others get the band mask (a folded global block none: block 1
  // with an unbounded window keeps every key)
  const int tq0 = 2 * bt - sb;
  const bool inner0 = tq0 >= 1 && kBlk * tq0 + kBlk - 1 <= c.W;
  const bool inner1 = tq0 + 1 >= 1 && kBlk * (tq0 + 1) + kBlk - 1 <= c.W;
  if (tt >= c.ngp && !(inner0 && inner1)) {
    band_mask(s0, gs0 ? 1 : tq0, gs0 ? 0x7fffffff : c.W);
    band_mask(s1, gs1 ? 1 : tq0 + 1, gs1 ? 0x7fffffff : c.W);
  }
  const float ms = cross_half_max(vmax(max16(s0), max16(s1))) * c2;
  if (__builtin_expect(__ballot(ms > m_run + kLazy) != 0ull, 0)) rescale(ms, o, m_run, l_run);
  v8 p0[2], p1[2];
  exp_p<T>(s0, m_run, c2, l_run, p0);
  exp_p<T>(s1, m_run, c2, l_run, p1);
  pv_frag<T>(vf0, p0, o);
  pv_frag<T>(vf1, p1, o);
  const int e = tt + kAhead;
  store_entry<T, RAW, ANY, PAST>(ring[ring_slot<FOLD>(e)], set, c, e);
  __builtin_amdgcn_sched_barrier(0);
  load_entry<T, ANY, PAST>(set, c, e + kDepth);
  if (BAR) __syncthreads();
}

// RAW: read the raw masks (else global_count and the shifted mask); ANY (with RAW):
// global tokens at any positions, through global_idx / global_count; GWG: workgroups
// past the band tiles compute the global rows, and the band tiles run no split.
// HELP (8 waves, at most 32 global tokens): four helper waves compute the tile's key
// split of the global rows beside the band waves (help_run), and the band waves run no
// split.
template <typename T, bool RAW, bool ANY, bool GWG, bool HELP>
__global__ __launch_bounds__(HELP ? kThreads + 64 * kHelp : kThreads)
__attribute__((amdgpu_waves_per_eu(HELP ? 3 : 2, HELP ? 3 : 2))) void attn_mfma_kernel(AttnArgs a, int n_tiles) {
  __shared__ __attribute__((aligned(16))) Slot<T> ring[kRing];
  __shared__ int s_nb;
  typedef typename Frag<T>::v8 v8;
  const int lane = lane_id();
  const int wave = wave_id();   // uniform: index math on the scalar unit
  const int rg = wave % kRowGroups, sb = wave / kRowGroups;
  const int n = lane & 31, g = lane >> 5;
  const int n_wg = a.B * a.H * n_tiles;
  if constexpr (GWG) {
    if ((int)blockIdx.x >= n_wg) {   // uniform: the whole workgroup
      global_rows_wg<T, RAW, ANY>(a, ring, (int)blockIdx.x - n_wg);
      return;
    }
  }
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
  c.ngp = (a.G + kEnt - 1) / kEnt;
  c.r0 = c.tile * kTile;
  c.kbase = c.r0 - (a.W >> 1);
  // a row group needs nband + 1 band blocks (its second sub-block starts one block
  // later): npb entries; the row groups' windows together span npb + kRowGroups - 1
  const int nband = (c.W + 2 * kBlk - 1) / kBlk;
  const int npb = (nband + 2) / 2;
  const int n_steps = c.ngp + npb;
  c.npb = npb;
  c.n_list = c.ngp + npb + kRowGroups - 1;
  // HELP: the one global-key entry is folded into the band steps (band_step), so the
  // loop runs steps kF .. n_steps - 1 (the list keeps the global entry as entry 0)
  constexpr int kF = HELP ? 1 : 0;
  const size_t head = (size_t)c.bh * c.S * 64;
  c.mask = (const T*)(RAW ? a.local_mask : a.bias) + (size_t)c.b * c.S;
  c.gi = ANY ? a.gidx + (size_t)c.b * c.S : nullptr;
  c.gm = ANY ? (const unsigned short*)a.global_mask + (size_t)c.b * c.S : nullptr;
  const float c2 = a.scale * kLog2e;
  if constexpr (HELP) {
    static_assert(kWaves == 8 && !GWG, "helper waves: 8-wave band tiles");
    __shared__ __attribute__((aligned(16))) HelpLds hl;
    if (wave >= kWaves) {   // uniform: the whole wave
      // the band waves execute the prologue barrier and one per pair of steps
      help_run<T, RAW, ANY>(a, c, 1 + (n_steps - kF) / 2, hl, &s_nb);
      return;
    }
  }
  const bool split = !GWG && !HELP && a.G > 0 && c.tile < a.n_split;
  // 4-wave layout: two workgroups share a CU, and the dispatcher places one on every
  // CU before it places a second, so workgroups of consecutive dispatch generations
  // (wg_per_gen workgroups each) pair up.  Odd generations run their split before the
  // band loop, even ones after it: one workgroup's memory round trips overlap the
  // other's band work.  (8 waves: one workgroup per CU, the split always runs last.)
  const bool sfirst = kWaves == 4 && split && a.wg_per_gen > 0 &&
                      (((int)blockIdx.x / a.wg_per_gen) & 1);
  c.split = split;
  c.split_tail = split && !sfirst;
  c.sp_lo = split ? c.tile * a.split_len : 0;
  c.sp_hi = split ? min(c.S, c.sp_lo + a.split_len) : 0;
  c.kh = (const T*)a.k + head;
  c.vh = (const T*)a.v + head;
  c.kgh = split ? (const T*)a.kg + head : c.kh;
  c.vgh = split ? (const T*)a.vg + head : c.vh;

  // every load the prologue needs is issued before anything waits: the global-mask
  // values, (split-first) the split's first round and its queries, the first ring
  // entries, Q, the register sets.  Only wave 0 counts the global tokens and hands
  // the count to the other waves at the prologue barrier.  (Every workgroup of a
  // batch row reads the same mask values: one request per workgroup instead of one
  // per wave keeps that cache line from becoming a hot spot.)
  // helper layout: a tile whose rows are all padding (or past S) has all-zero output;
  // its band waves skip the loop and keep only its barriers (the helper waves still
  // compute the tile's key split of the global rows on their schedule)
  __shared__ int s_live[kWaves];
  bool tile_dead = false;
  const bool counter = wave == 0;
  const int gfirst = counter ? count_load<T, RAW, ANY>(a, c.b) : 0;
  __builtin_amdgcn_sched_barrier(0);
  Stage<T> spl[kSplitEnt];
  v8 qg0[4];
  if (sfirst) {
    const uint32_t bytes = (uint32_t)c.S * 128u;
    const rsrc_t rkg = make_rsrc(c.kgh, bytes), rvg = make_rsrc(c.vgh, bytes);
    const rsrc_t rm = make_rsrc(c.mask, (uint32_t)c.S * 2u);
#pragma unroll
    for (int e = 0; e < kSplitEnt; ++e) stage_load<T>(spl[e], rkg, rvg, rm, c.sp_lo + kEnt * e);
    load_q<T>(qg0, (const T*)a.qg + ((size_t)c.bh * a.G + (n < a.G ? n : 0)) * 64, n < a.G);
  }
  __builtin_amdgcn_sched_barrier(0);
  Stage<T> pro[kAhead + kF];
#pragma unroll
  for (int i = 0; i < kAhead + kF; ++i) load_entry<T, ANY, true>(pro[i], c, i);
  // Q before the register sets: in the loop its wait count then never holds back
  // the sets in flight
  v8 qf[4];
  const int srow = c.r0 + 64 * rg + 32 * sb + n;
  load_q<T>(qf, (const T*)a.q + head + (size_t)(srow < c.S ? srow : 0) * 64, srow < c.S);
  // the row's mask value (and global flag) for the epilogue, loaded now so that no
  // load sits between the band loop and the output stores
  const int srow_c = srow < c.S ? srow : 0;
  const T row_mask = c.mask[srow_c];
  const unsigned short row_gflag = ANY ? c.gm[srow_c] : (unsigned short)0;
  __builtin_amdgcn_sched_barrier(0);
  static_assert(kDepth == 2, "steps run in pairs: entry e uses set e % 2");
  // after the band loop the ring holds list entries up to n_list + kStaged - 1 and the
  // register sets the next kDepth: the split's first round is n_list .. n_list +
  // kSplitEnt - 1, its last kSplitEnt - kStaged entries still in registers
  constexpr int kStaged = kAhead - (kRowGroups - 1);
  static_assert(kStaged >= 1 && kSplitEnt - kStaged >= 1 && kSplitEnt - kStaged <= kDepth,
                "split round = entries staged by the band loop + entries in the register sets");
  Stage<T> st[kDepth];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) {
    load_entry<T, ANY, true>(st[(kAhead + kF + u) % kDepth], c, kAhead + kF + u);
    __builtin_amdgcn_sched_barrier(0);
  }
  c.nb = counter ? count_globals<T, RAW, ANY>(a, c.b, gfirst) : 0;
  int ticket = 0;
  if constexpr (kWaves == 8) {
    // the first entries are written before the prologue barrier (wave 0 alone writes
    // the per-key terms, with its own count)
#pragma unroll
    for (int i = 0; i < kAhead + kF; ++i)
      store_entry<T, RAW, ANY, true>(ring[ring_slot<HELP>(i)], pro[i], c, i);
    if (counter && lane == 0) s_nb = c.nb;
    if constexpr (HELP) {
      // does any of the wave's rows exist and carry a live mask value?
      const bool wlive = __ballot(srow < c.S && mask_live<RAW>(Elem<T>::to_f(row_mask))) != 0ull;
      if (lane == 0) s_live[wave] = wlive ? 1 : 0;
    }
    __syncthreads();
    c.nb = __builtin_amdgcn_readfirstlane(s_nb);
    if constexpr (HELP) {
      int any = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) any |= s_live[w];
      tile_dead = __builtin_amdgcn_readfirstlane(any) == 0;
    }
  } else {
    if (counter && lane == 0) s_nb = c.nb;
    __syncthreads();
    c.nb = __builtin_amdgcn_readfirstlane(s_nb);
    // split first: its round is in the ring's slots 0 .. kSplitEnt - 1 (its wave
    // states in the others), then the partial is published and the ticket taken; the
    // band entries go in afterwards
    if (sfirst && c.nb > 0) {
#pragma unroll
      for (int e = 0; e < kSplitEnt; ++e)
        stage_store<T, RAW>(ring[e], spl[e], c.sp_lo + kEnt * e, c.sp_lo, c.sp_hi);
      global_split_run<T, RAW, ANY, true>(a, c, c.tile, ring, 0, qg0);
      ticket = take_ticket<T>(a, c);
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) store_entry<T, RAW, ANY, true>(ring[i], pro[i], c, i);
    __syncthreads();
  }
  const bool do_split = split && c.nb > 0;

  f32x16 o[2] = {f32x16{}, f32x16{}};
  float m_run = kNegBig, l_run = 0.0f;
  constexpr int s0i = (kAhead + kF) % kDepth, s1i = (kAhead + kF + 1) % kDepth;
  // Barriers: 8 waves, one per pair of steps (an entry written at step t is read from
  // step t + 2 on; the slot it overwrites, entry t - 3's, was last read before the
  // previous barrier); 4 waves, one per step (written at t, read from t + 1; the slot
  // it overwrites, entry t - 2's, was last read at step t - 2).  Steps t < n_plain
  // stage and load entries of the list only; on split-last tiles the later ones reach
  // past it (the split's first round)
  constexpr bool kBar0 = !kPairs;
  const int n_plain = c.split_tail ? c.n_list - kAhead - kDepth : n_steps;
  int t0 = kF;
  if (HELP && tile_dead) {
    for (int i = 0; i < (n_steps - kF) / 2; ++i) __syncthreads();
    t0 = n_steps;
  }
  for (; t0 + 2 <= n_plain; t0 += 2) {
    band_step<T, RAW, ANY, false, kBar0, HELP, HELP>(c, ring, t0, rg, sb, c2, st[s0i], qf, o, m_run, l_run);
    band_step<T, RAW, ANY, false, true, HELP, HELP>(c, ring, t0 + 1, rg, sb, c2, st[s1i], qf, o, m_run, l_run);
  }
  for (; t0 + 2 <= n_steps; t0 += 2) {
    band_step<T, RAW, ANY, true, kBar0, HELP, HELP>(c, ring, t0, rg, sb, c2, st[s0i], qf, o, m_run, l_run);
    band_step<T, RAW, ANY, true, true, HELP, HELP>(c, ring, t0 + 1, rg, sb, c2, st[s1i], qf, o, m_run, l_run);
  }
  if (t0 < n_steps)
    band_step<T, RAW, ANY, true, kBar0, HELP, HELP>(c, ring, t0, rg, sb, c2, st[s0i], qf, o, m_run, l_run);

  // the split's queries (rows 0 .. 31 below G; rows from n_b on are computed but not
  // published) go out before the epilogue, which hides their latency
  const bool tail = do_split && !sfirst;
  if (tail)
    load_q<T>(qg0, (const T*)a.qg + ((size_t)c.bh * a.G + (n < a.G ? n : 0)) * 64, n < a.G);

  // epilogue: normalise and store the local rows
  auto epilogue = [&]() {
    typedef typename Frag<T>::v4 v4;
    const float l_tot = cross_half_sum(l_run);
    // global rows are written by the combine
    const bool local = srow < c.S && (ANY ? (row_gflag & 0x7fff) != 0 : srow >= c.nb);
    const bool live = mask_live<RAW>(Elem<T>::to_f(row_mask));
    const float inv = live ? 1.0f / l_tot : 0.0f;
    T* dst = (T*)a.out + (size_t)c.b * a.out_sb + (size_t)c.h * a.out_sh + (size_t)srow * a.out_ss;
    // lanes n and n + 32 hold alternate groups of 4 dims of one row; each sends the
    // other the group it lacks (every lane active), so that lane (n, 0) stores dims
    // 16p .. 16p + 7 and lane (n, 1) dims 16p + 8 .. 16p + 15 of each 32-dim half as
    // one 16-byte store: half the store instructions, 32 contiguous bytes per row each
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        v4 x, y;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = Elem<T>::from_f(live ? o[mb][8 * p + i] * inv : 0.0f);
          y[i] = Elem<T>::from_f(live ? o[mb][8 * p + 4 + i] * inv : 0.0f);
        }
        const u32x2 xb = __builtin_bit_cast(u32x2, x), yb = __builtin_bit_cast(u32x2, y);
        const u32x2 sd = g ? xb : yb;
        const u32x2 rb = {(uint32_t)__shfl_xor((int)sd[0], 32), (uint32_t)__shfl_xor((int)sd[1], 32)};
        const u32x4 w = g ? u32x4{rb[0], rb[1], yb[0], yb[1]} : u32x4{xb[0], xb[1], rb[0], rb[1]};
        if (local) *(u32x4*)(dst + 32 * mb + 16 * p + 8 * g) = w;
      }
    }
  };

  // split last, before the output stores: the ticket waits for every store of the wave
  // to complete, so the partial is published and the ticket taken while no output
  // store is in flight yet (the band accumulators stay in registers meanwhile); list
  // entries n_list .. n_list + kStaged - 1 are in the ring, the rest of the round in
  // the register sets
  if (!tail) epilogue();
  if (tail) {
    __syncthreads();   // band reads done
    // entry e sits in set e % 2: a uniform branch keeps the set index static (an
    // index known only at run time would put the sets in scratch memory)
    const int ef = c.n_list + kStaged;
    if constexpr (kSplitEnt - kStaged == 2) {
      if ((ef & 1) == 0) {
        store_entry<T, RAW, ANY, true>(ring[ef % kRing], st[0], c, ef);
        store_entry<T, RAW, ANY, true>(ring[(ef + 1) % kRing], st[1], c, ef + 1);
      } else {
        store_entry<T, RAW, ANY, true>(ring[ef % kRing], st[1], c, ef);
        store_entry<T, RAW, ANY, true>(ring[(ef + 1) % kRing], st[0], c, ef + 1);
      }
    } else {
      if ((ef & 1) == 0)
        store_entry<T, RAW, ANY, true>(ring[ef % kRing], st[0], c, ef);
      else
        store_entry<T, RAW, ANY, true>(ring[ef % kRing], st[1], c, ef);
    }
    __syncthreads();
    global_split_run<T, RAW, ANY, true>(a, c, c.tile, ring, c.n_list % kRing, qg0);
    ticket = take_ticket<T>(a, c);
    epilogue();
  }
  // the workgroup whose ticket completed the (b, h) merges the partials
  if (do_split) {
    __shared__ int s_last;
    if (threadIdx.x == 0) s_last = ticket == a.n_split - 1;
    __syncthreads();
    if (s_last) global_combine<T, RAW, ANY>(a, c);
  }
}

#if !defined(LF_ATTN_GWG_TU) && !defined(LF_ATTN_W4_TU)
static_assert(kWaves == 8, "the main translation unit holds the 8-wave layout");

// Compute units of the current device (cached per device).
int cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  return n;
}

// The 4-wave layout for sequences of at least 8192 tokens, where its overlap of two
// workgroups per CU gains more than its extra band-halo staging costs (measured: 3 to
// 21 % faster from S = 8192 on, up to 20 % slower at S = 4096).  LF_ATTN_WAVES=4 or 8
// (read on every call) forces a layout.
bool layout_w4(int S) {
  const char* f = getenv("LF_ATTN_WAVES");
  if (f && f[0] == '4' && f[1] == 0) return true;
  if (f && f[0] == '8' && f[1] == 0) return false;
  return S >= 8192;
}

template <typename T>
hipError_t launch_t(const AttnArgs& args, hipStream_t st) {
  const int n_tiles = (args.S + kTile - 1) / kTile;
  const int64_t band = (int64_t)args.B * args.H * n_tiles;
  // band tiles that leave CUs idle: the global rows of each (b, h) get a workgroup of
  // their own (one split over all keys) that runs beside them
  AttnArgs a = args;
  // LF_ATTN_NO_GWG=1 (read on every call) keeps the split path on small grids too
  const char* no_gwg = getenv("LF_ATTN_NO_GWG");
  const bool gwg = a.G > 0 && band + (int64_t)a.B * a.H <= cu_count() &&
                   !(no_gwg && no_gwg[0] == '1');
  const bool w4 = !gwg && layout_w4(a.S);
  // helper waves for the global rows: one query block (G <= 32), one 256-key split per
  // tile, and at least three barriers in the band loop's schedule for their phases
  // (LF_ATTN_NO_HELP=1, read on every call, keeps the band tiles' own split)
  // (with helpers the global-key entry is folded into the band steps: npb steps)
  const int npb = ((a.W + 2 * kBlk - 1) / kBlk + 2) / 2;
  const char* no_help = getenv("LF_ATTN_NO_HELP");
  const bool help = !gwg && !w4 && (!a.any_pos || a.raw) && a.G > 0 && a.G <= 32 &&
                    a.split_len == kHelp * kHelpKeys &&
                    1 + npb / 2 >= 3 && !(no_help && no_help[0] == '1');
  if (gwg) {
    a.n_split = 1;
    a.split_len = (a.S + kBlk * kWaves - 1) / (kBlk * kWaves) * (kBlk * kWaves);
  }
  a.wg_per_gen = cu_count();
  const int64_t grid = band + (gwg ? (int64_t)a.B * a.H : 0);
  if (!w4) {
    if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (a.G > 0 && (a.split_len % (kBlk * kWaves) != 0 || a.n_split > n_tiles))
      return hipErrorInvalidConfiguration;
  }
  if ((int64_t)a.S * 128 > 0x7fffffff) return hipErrorInvalidValue;   // per-head buffer range
  if (a.ev_begin) {
    hipError_t e0 = hipEventRecord(a.ev_begin, st);
    if (e0 != hipSuccess) return e0;
  }
  if (w4) {
    // the 4-wave layout, instantiated in a translation unit of its own
    // (attn_mfma_w4.hip); it checks its own grid and split plan
    const hipError_t ew = launch_attention_w4(a, st);
    if (ew != hipSuccess) return ew;
  } else if (gwg) {
    // instantiated in a translation unit of its own (attn_mfma_gwg.hip), so that the
    // code of the kernels below does not change with it
    const hipError_t eg = launch_attention_gwg(a, n_tiles, (unsigned)grid, st);
    if (eg != hipSuccess) return eg;
  } else if (help) {
    constexpr int kHT = kThreads + 64 * kHelp;
    if (a.raw && a.any_pos)
      attn_mfma_kernel<T, true, true, false, true><<<(unsigned)grid, kHT, 0, st>>>(a, n_tiles);
    else if (a.raw)
      attn_mfma_kernel<T, true, false, false, true><<<(unsigned)grid, kHT, 0, st>>>(a, n_tiles);
    else
      attn_mfma_kernel<T, false, false, false, true><<<(unsigned)grid, kHT, 0, st>>>(a, n_tiles);
  } else if (a.raw && a.any_pos) {
    attn_mfma_kernel<T, true, true, false, false><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles);
  } else if (a.raw) {
    attn_mfma_kernel<T, true, false, false, false><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles);
  } else {
    attn_mfma_kernel<T, false, false, false, false><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_end) e = hipEventRecord(a.ev_end, st);
  return e;
}
#elif defined(LF_ATTN_GWG_TU)
template <typename T>
void launch_gwg_t(const AttnArgs& a, int n_tiles, unsigned grid, hipStream_t st) {
  if (a.raw && a.any_pos)
    attn_mfma_kernel<T, true, true, true, false><<<grid, kThreads, 0, st>>>(a, n_tiles);
  else if (a.raw)
    attn_mfma_kernel<T, true, false, true, false><<<grid, kThreads, 0, st>>>(a, n_tiles);
  else
    attn_mfma_kernel<T, false, false, true, false><<<grid, kThreads, 0, st>>>(a, n_tiles);
}
#else
static_assert(kWaves == 4, "attn_mfma_w4.hip holds the 4-wave layout");
template <typename T>
hipError_t launch_w4_t(const AttnArgs& a, hipStream_t st) {
  const int n_tiles = (a.S + kTile - 1) / kTile;
  const int64_t grid = (int64_t)a.B * a.H * n_tiles;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.G > 0 && (a.split_len % (kBlk * kWaves) != 0 || a.n_split > n_tiles))
    return hipErrorInvalidConfiguration;
  if (a.raw && a.any_pos)
    attn_mfma_kernel<T, true, true, false, false><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles);
  else if (a.raw)
    attn_mfma_kernel<T, true, false, false, false><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles);
  else
    attn_mfma_kernel<T, false, false, false, false><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles);
  return hipGetLastError();
}
#endif

}  // namespace

#if !defined(LF_ATTN_GWG_TU) && !defined(LF_ATTN_W4_TU)
void attn_split_plan(int S, int* n_split, int* split_len) {
  // one split per tile (256 rows, or 128 in the 4-wave layout), at most 32 splits per
  // (b, h); splits are whole rounds of (waves x 32) keys
  const bool w4 = layout_w4(S);
  const int tile = w4 ? kTile / 2 : kTile;
  const int unit = w4 ? kBlk * kWaves / 2 : kBlk * kWaves;
  const int n_tiles = (S + tile - 1) / tile;
  const int want = n_tiles < kMaxSplit ? n_tiles : kMaxSplit;
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

#elif defined(LF_ATTN_GWG_TU)
hipError_t launch_attention_gwg(const AttnArgs& a, int n_tiles, unsigned grid, hipStream_t st) {
  switch (a.dtype) {
    case 1: launch_gwg_t<f16>(a, n_tiles, grid, st); return hipGetLastError();
    case 2: launch_gwg_t<bf16>(a, n_tiles, grid, st); return hipGetLastError();
  }
  return hipErrorInvalidValue;
}
#else
hipError_t launch_attention_w4(const AttnArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 1: return launch_w4_t<f16>(a, st);
    case 2: return launch_w4_t<bf16>(a, st);
  }
  return hipErrorInvalidValue;
}
#endif

}  // namespace lf
