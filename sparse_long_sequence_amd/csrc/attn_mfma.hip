// fp16 / bf16 band + global attention on the gfx950 matrix cores.
//
// [FT-LF] = the page "FasterTransformer Longformer 推理加速实践：PyTorch 集成、输入约束与
// 端到端性能解析", section "Longformer Encoder 计算流程":
//   per-layer step 3  local sliding-window attention plus global attention;
//   per-layer step 4  one masked softmax: a local token normalises over its window
//                     and the global tokens, a global token over the whole
//                     sequence, padded rows are zeroed;
//   preprocessing 2   the shifted local mask is an additive score bias.
// The page's own design (three window-GEMM segments with score buffers, then a
// separate softmax kernel) is not followed: here scores never leave registers.
//
// Work split (one launch, two kinds of 256-thread workgroups):
//  * band workgroup = 128 query rows of one (b, h), 32 per wave.  Keys stream
//    through LDS in 64-row chunks, double-buffered: first the global keys
//    (gathered through global_idx), then the band [max(n_b, t0-W/2),
//    min(S-1, t0+127+W/2)].  K is kept row-major, V is written transposed so
//    both MFMA operands read contiguous 8-element fragments.
//  * global workgroup = one key split of one (b, h) for up to 64 global rows;
//    each wave streams its own 64-key chunks (K straight from memory into MFMA
//    fragments, V through a per-wave transposed LDS tile), the four wave states
//    are merged in LDS and one partial (m, l, o[64]) per row goes to the
//    workspace; a small combine kernel merges the splits.
//
// Per chunk and wave: S^T = K Q^T (8 x v_mfma_f32_32x32x16), so each lane holds
// 32 scores of ONE query; row max = in-lane max + one lane^32 exchange; the
// online-softmax state (m in log2 units, l, O^T) is per lane; the running max is
// only moved when it grows by more than 8 (p <= 2^8 then, exact in fp16/bf16 range),
// so rescaling the 32 O^T accumulators is rare; P is rounded to the input type and
// its row sum is taken from the rounded values (v_dot2), then O^T += V^T P^T
// (8 more MFMAs).
#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

namespace {

constexpr int kChunk = 64;
constexpr int kKld = 72;   // LDS row pitch of K (elements): 144 B, conflict-free 16 B reads
constexpr int kVld = 68;   // LDS row pitch of V^T (elements): 136 B, conflict-free 8 B reads
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;   // running-max start: finite, so exp2 never sees inf-inf
constexpr float kLazy = 8.0f;         // rescale only when the max grows by more than 2^8
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTileRows = 32 * kWaves;

template <typename T>
struct ChunkBuf {
  T k[kChunk * kKld];
  T vt[64 * kVld];
  float bias2[kChunk];   // key bias * log2(e); -inf for empty slots
  int flag;              // nonzero: some slot has a nonzero bias
  int pad[3];
};

template <typename T>
struct WaveBuf {
  T vt[64 * kVld];
  float bias2[kChunk];
};

// ---------------------------------------------------------------- staging (band)
template <typename T>
struct StageRegs {
  u32x4 k0, k1, v0, v1;
  float bias2;
};

// Thread t stages rows 2*(t/8) and 2*(t/8)+1, columns 8*(t%8)..+7, of the chunk;
// threads 0..63 also stage the key bias of slot t.
template <typename T>
__device__ inline void stage_load(StageRegs<T>& r, const T* __restrict__ kh,
                                  const T* __restrict__ vh, const T* __restrict__ bias_row,
                                  const int32_t* __restrict__ gidx, bool gather, int first,
                                  int count, int S) {
  const int t = threadIdx.x;
  const int rp = t >> 3, col = t & 7;
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int slot = 2 * rp + e;
    int key = -1;
    if (slot < count) key = gather ? gidx[first + slot] : first + slot;
    const bool ok = key >= 0 && key < S;
    u32x4 kk = zero, vv = zero;
    if (ok) {
      kk = *(const u32x4*)(kh + (size_t)key * 64 + col * 8);
      vv = *(const u32x4*)(vh + (size_t)key * 64 + col * 8);
    }
    if (e == 0) { r.k0 = kk; r.v0 = vv; } else { r.k1 = kk; r.v1 = vv; }
  }
  if (t < kChunk) {
    int key = -1;
    if (t < count) key = gather ? gidx[first + t] : first + t;
    r.bias2 = (key >= 0 && key < S) ? Elem<T>::to_f(bias_row[key]) * kLog2e : -INFINITY;
  }
}

template <typename T>
__device__ inline void stage_store(ChunkBuf<T>& buf, const StageRegs<T>& r) {
  const int t = threadIdx.x;
  const int rp = t >> 3, col = t & 7;
  *(u32x4*)&buf.k[(2 * rp) * kKld + col * 8] = r.k0;
  *(u32x4*)&buf.k[(2 * rp + 1) * kKld + col * 8] = r.k1;
  // transpose: element e of rows (2rp, 2rp+1) -> V^T[8col+e][2rp..2rp+1] as one dword
  const uint32_t* a = (const uint32_t*)&r.v0;
  const uint32_t* b = (const uint32_t*)&r.v1;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (a[w] & 0xffffu) | (b[w] << 16);
    const uint32_t hi = (a[w] >> 16) | (b[w] & 0xffff0000u);
    *(uint32_t*)&buf.vt[(col * 8 + 2 * w) * kVld + 2 * rp] = lo;
    *(uint32_t*)&buf.vt[(col * 8 + 2 * w + 1) * kVld + 2 * rp] = hi;
  }
  if (t < kChunk) {
    buf.bias2[t] = r.bias2;
    const uint64_t any = __ballot(r.bias2 != 0.0f);
    if (t == 0) buf.flag = any != 0ull;
  }
}

// ---------------------------------------------------------------- per-wave math
template <typename T>
struct Frags {
  typedef typename Elem<T>::vec8 v8;
  typedef typename Elem<T>::vec4 v4;
  typedef typename Elem<T>::vec2 v2;
};

// Scores -> probabilities for one chunk, update of the lane's online-softmax state,
// and the P^T operand fragments for the PV product.
template <typename T, bool MASK, bool BIAS>
__device__ inline void softmax_chunk(f32x16& s0, f32x16& s1, const float* __restrict__ bias2,
                                     int key0, int srow, int half, int S, float c2,
                                     float& m_run, float& l_run, f32x16* o, int n_o,
                                     typename Frags<T>::v8 pf[4]) {
  const int g = lane_id() >> 5;
  float x[32];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    x[v] = s0[v] * c2;
    x[16 + v] = s1[v] * c2;
  }
  if (BIAS) {
#pragma unroll
    for (int q4 = 0; q4 < 8; ++q4) {
      const int kl = (q4 >> 2) * 32 + (q4 & 3) * 8 + 4 * g;
      const f32x4 bb = *(const f32x4*)&bias2[kl];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * q4 + i] += bb[i];
    }
  }
  if (MASK) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int kl = (e >> 4) * 32 + ((e & 15) >> 2) * 8 + 4 * g + (e & 3);
      const int j = key0 + kl;
      const bool ok = (j - srow <= half) && (srow - j <= half) && (j < S);
      x[e] = ok ? x[e] : -INFINITY;
    }
  }
  float mx = x[0];
#pragma unroll
  for (int e = 1; e < 32; ++e) mx = fmaxf(mx, x[e]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const bool need = mx > m_run + kLazy;
  if (__ballot(need)) {
    const float m_new = need ? mx : m_run;
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
    for (int i = 0; i < n_o; ++i) o[i] *= alpha;
    m_run = m_new;
  }
  typedef typename Frags<T>::v2 v2;
  float lsum = 0.0f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const int e = 16 * (s >> 1) + 8 * (s & 1) + i;
      const T p0 = Elem<T>::from_f(fast_exp2(x[e] - m_run));
      const T p1 = Elem<T>::from_f(fast_exp2(x[e + 1] - m_run));
      pf[s][i] = p0;
      pf[s][i + 1] = p1;
      v2 pp = {p0, p1};
      lsum = dot2_ones(pp, lsum);
    }
  }
  l_run += lsum;
}

// O^T[mb] += V^T P^T over one chunk; V^T rows (d) in LDS with pitch kVld.
template <typename T>
__device__ inline void pv_chunk(const T* __restrict__ vt, const typename Frags<T>::v8 pf[4],
                                f32x16 o[2]) {
  typedef typename Frags<T>::v8 v8;
  typedef typename Frags<T>::v4 v4;
  const int n = lane_id() & 31, g = lane_id() >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const T* row = vt + (32 * mb + n) * kVld + 16 * s + 4 * g;
      const v4 lo = *(const v4*)row;
      const v4 hi = *(const v4*)(row + 8);
      const v8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[mb] = mfma32(va, pf[s], o[mb]);
    }
  }
}

// S^T for a chunk whose K rows sit in LDS (pitch kKld).
template <typename T>
__device__ inline void qk_chunk_lds(const T* __restrict__ k, const typename Frags<T>::v8 qf[4],
                                    f32x16& s0, f32x16& s1) {
  typedef typename Frags<T>::v8 v8;
  const int n = lane_id() & 31, g = lane_id() >> 5;
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v8 a0 = *(const v8*)&k[n * kKld + 16 * t + 8 * g];
    const v8 a1 = *(const v8*)&k[(32 + n) * kKld + 16 * t + 8 * g];
    s0 = mfma32(a0, qf[t], s0);
    s1 = mfma32(a1, qf[t], s1);
  }
}

template <typename T>
__device__ inline void store_rows(const AttnArgs& a, int b, int h, int srow, bool write,
                                  bool live, const f32x16 o[2], float l_tot) {
  if (!write) return;
  const int g = lane_id() >> 5;
  T* dst = (T*)a.out + (size_t)b * a.out_sb + (size_t)h * a.out_sh + (size_t)srow * a.out_ss;
  const float inv = live ? 1.0f / l_tot : 0.0f;
  typedef typename Frags<T>::v4 v4;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = Elem<T>::from_f(live ? o[mb][4 * j + i] * inv : 0.0f);
      *(v4*)(dst + 32 * mb + 8 * j + 4 * g) = w;
    }
  }
}

// ---------------------------------------------------------------- band workgroup
template <typename T>
__device__ void band_tile(const AttnArgs& a, int bh, int tile, ChunkBuf<T>* bufs) {
  typedef typename Frags<T>::v8 v8;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int b = bh / a.H, h = bh % a.H;
  const int S = a.S, half = a.W >> 1;
  const int nb = a.gcnt[b];
  const int t0 = tile * kTileRows;
  const int tlo = max(t0, nb), thi = min(t0 + kTileRows - 1, S - 1);
  if (tlo > thi) return;   // whole tile is global rows: written by the global path
  const int row0 = t0 + 32 * wave;
  const int srow = row0 + n;
  const int r_lo = max(row0, nb), r_hi = min(row0 + 31, S - 1);
  const bool wave_active = r_lo <= r_hi;

  const size_t head = (size_t)bh * S * 64;
  const T* qh = (const T*)a.q + head;
  const T* kh = (const T*)a.k + head;
  const T* vh = (const T*)a.v + head;
  const T* bias_row = (const T*)a.bias + (size_t)b * S;
  const int32_t* gidx = a.gidx + (size_t)b * S;

  v8 qf[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (srow < S)
      qf[t] = *(const v8*)(qh + (size_t)srow * 64 + 16 * t + 8 * g);
    else
      qf[t] = v8{};
  }
  const int n_g = (nb + kChunk - 1) / kChunk;
  const int lo = max(nb, tlo - half), hi = min(S - 1, thi + half);
  const int n_b = (hi - lo + kChunk) / kChunk;
  const int total = n_g + n_b;
  const float c2 = a.scale * kLog2e;

  f32x16 o[2] = {f32x16{}, f32x16{}};
  float m_run = kNegBig, l_run = 0.0f;

  auto chunk_first = [&](int c) { return c < n_g ? c * kChunk : lo + (c - n_g) * kChunk; };
  auto chunk_count = [&](int c) {
    return c < n_g ? min(kChunk, nb - c * kChunk) : min(kChunk, hi - chunk_first(c) + 1);
  };

  StageRegs<T> r;
  stage_load<T>(r, kh, vh, bias_row, gidx, 0 < n_g, chunk_first(0), chunk_count(0), S);
  stage_store<T>(bufs[0], r);
  __syncthreads();
  for (int c = 0; c < total; ++c) {
    const bool more = c + 1 < total;
    if (more)
      stage_load<T>(r, kh, vh, bias_row, gidx, c + 1 < n_g, chunk_first(c + 1),
                    chunk_count(c + 1), S);
    ChunkBuf<T>& cb = bufs[c & 1];
    if (wave_active) {
      const bool is_band = c >= n_g;
      const int kb = chunk_first(c);
      bool touch = true, interior = true;
      if (is_band) {
        touch = kb <= r_hi + half && kb + kChunk - 1 >= r_lo - half;
        interior = kb >= r_hi - half && kb + kChunk - 1 <= r_lo + half && kb + kChunk - 1 < S;
      }
      if (touch) {
        f32x16 s0, s1;
        qk_chunk_lds<T>(cb.k, qf, s0, s1);
        v8 pf[4];
        const bool bias = cb.flag != 0;
        if (interior) {
          if (bias)
            softmax_chunk<T, false, true>(s0, s1, cb.bias2, kb, srow, half, S, c2, m_run, l_run,
                                          o, 2, pf);
          else
            softmax_chunk<T, false, false>(s0, s1, cb.bias2, kb, srow, half, S, c2, m_run,
                                           l_run, o, 2, pf);
        } else {
          if (bias)
            softmax_chunk<T, true, true>(s0, s1, cb.bias2, kb, srow, half, S, c2, m_run, l_run,
                                         o, 2, pf);
          else
            softmax_chunk<T, true, false>(s0, s1, cb.bias2, kb, srow, half, S, c2, m_run, l_run,
                                          o, 2, pf);
        }
        pv_chunk<T>(cb.vt, pf, o);
      }
    }
    if (more) stage_store<T>(bufs[(c + 1) & 1], r);
    __syncthreads();
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const bool write = srow < S && srow >= nb;
  const bool live = write && Elem<T>::to_f(bias_row[write ? srow : 0]) == 0.0f;
  store_rows<T>(a, b, h, srow, write, live, o, l_tot);
}

// ---------------------------------------------------------------- global workgroup
// Rows r_base .. r_base + 32*NQB - 1 of the global queries of (b, h), keys of one split.
template <typename T, int NQB>
__device__ void global_split(const AttnArgs& a, int bh, int split, int qgroup, char* smem) {
  typedef typename Frags<T>::v8 v8;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int b = bh / a.H, h = bh % a.H;
  const int S = a.S;
  const int nb = a.gcnt[b];
  const int r_base = qgroup * 32 * NQB;
  if (r_base >= nb) return;
  const int k0 = split * a.split_len;
  const int k1 = min(S, k0 + a.split_len);

  const size_t head = (size_t)bh * S * 64;
  const T* kh = (const T*)a.kg + head;
  const T* vh = (const T*)a.vg + head;
  const T* qgh = (const T*)a.qg + (size_t)bh * a.G * 64;
  const T* bias_row = (const T*)a.bias + (size_t)b * S;
  WaveBuf<T>* wb = (WaveBuf<T>*)smem + wave;

  v8 qf[NQB][4];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = r_base + 32 * qb + n;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      qf[qb][t] = r < nb ? *(const v8*)(qgh + (size_t)r * 64 + 16 * t + 8 * g) : v8{};
  }
  f32x16 o[NQB][2];
  float m_run[NQB], l_run[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    o[qb][0] = f32x16{};
    o[qb][1] = f32x16{};
    m_run[qb] = kNegBig;
    l_run[qb] = 0.0f;
  }
  const float c2 = a.scale * kLog2e;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int kb = k0 + kChunk * wave; kb < k1; kb += kChunk * kWaves) {
    // K fragments straight from memory: lane (key n (+32), d-half g)
    v8 ka[2][4];
#pragma unroll
    for (int kblk = 0; kblk < 2; ++kblk) {
      const int key = kb + 32 * kblk + n;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        ka[kblk][t] = key < k1 ? *(const v8*)(kh + (size_t)key * 64 + 16 * t + 8 * g) : v8{};
    }
    // V chunk -> transposed per-wave LDS tile
    u32x4 va[4], vb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int task = lane + 64 * i;
      const int rp = task >> 3, col = task & 7;
      const int key = kb + 2 * rp;
      va[i] = key < k1 ? *(const u32x4*)(vh + (size_t)key * 64 + col * 8) : zero;
      vb[i] = key + 1 < k1 ? *(const u32x4*)(vh + (size_t)(key + 1) * 64 + col * 8) : zero;
    }
    const int bkey = kb + lane;
    const float bias2 = bkey < k1 ? Elem<T>::to_f(bias_row[bkey]) * kLog2e : -INFINITY;
    const bool any_bias = __ballot(bias2 != 0.0f) != 0ull;
    __builtin_amdgcn_wave_barrier();   // previous chunk's LDS reads issued before rewriting
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int task = lane + 64 * i;
      const int rp = task >> 3, col = task & 7;
      const uint32_t* pa = (const uint32_t*)&va[i];
      const uint32_t* pb = (const uint32_t*)&vb[i];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *(uint32_t*)&wb->vt[(col * 8 + 2 * w) * kVld + 2 * rp] = (pa[w] & 0xffffu) | (pb[w] << 16);
        *(uint32_t*)&wb->vt[(col * 8 + 2 * w + 1) * kVld + 2 * rp] =
            (pa[w] >> 16) | (pb[w] & 0xffff0000u);
      }
    }
    wb->bias2[lane] = bias2;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s0 = mfma32(ka[0][t], qf[qb][t], s0);
        s1 = mfma32(ka[1][t], qf[qb][t], s1);
      }
      v8 pf[4];
      if (any_bias)
        softmax_chunk<T, false, true>(s0, s1, wb->bias2, kb, 0, 0, S, c2, m_run[qb], l_run[qb],
                                      o[qb], 2, pf);
      else
        softmax_chunk<T, false, false>(s0, s1, wb->bias2, kb, 0, 0, S, c2, m_run[qb], l_run[qb],
                                       o[qb], 2, pf);
      pv_chunk<T>(wb->vt, pf, o[qb]);
    }
    (void)zero;
  }
  // merge the four wave states in LDS (reusing the per-wave tiles), then write one
  // partial (m, l, o[64]) per valid row
  float* mbuf = (float*)smem;   // [NQB*32][66]
  __syncthreads();
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int q = 32 * qb + n;
        float* row = mbuf + q * 66;
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
        float mm = m_run[qb], ll = l_tot, f_old = 0.0f, f_new = 1.0f;
        if (w > 0) {
          const float m_old = row[0];
          mm = fmaxf(m_old, m_run[qb]);
          f_old = fast_exp2(m_old - mm);
          f_new = fast_exp2(m_run[qb] - mm);
          ll = row[1] * f_old + l_tot * f_new;
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int d = 32 * mb + 8 * (v >> 2) + 4 * g + (v & 3);
            const float prev = w > 0 ? row[2 + d] : 0.0f;
            row[2 + d] = prev * f_old + o[qb][mb][v] * f_new;
          }
        if (g == 0) {
          row[0] = mm;
          row[1] = ll;
        }
      }
    }
    __syncthreads();
  }
  // 256 threads write NQB*32 rows x 66 floats
  const int rows = min(32 * NQB, nb - r_base);
  float* dst = a.partials + ((size_t)bh * a.n_split + split) * (size_t)a.G * 66 + (size_t)r_base * 66;
  for (int i = threadIdx.x; i < rows * 66; i += kThreads) dst[i] = mbuf[i];
}

// XCD-aware order: consecutive workgroup ids go round-robin over the 8 XCDs, so
// give each XCD a contiguous run of logical tiles (neighbouring tiles of one head
// share K/V rows in that XCD's L2).
__device__ inline int xcd_remap(int i, int n) {
  const int per = n / 8;
  const int full = per * 8;
  if (i >= full) return i;
  return (i % 8) * per + i / 8;
}

template <typename T, int NQB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma_kernel(AttnArgs a, int n_tiles,
                                                             int n_global_wg, int n_qgroups) {
  __shared__ __attribute__((aligned(16))) char smem[2 * sizeof(ChunkBuf<T>)];
  static_assert(kWaves * sizeof(WaveBuf<T>) <= 2 * sizeof(ChunkBuf<T>), "lds");
  static_assert(NQB * 32 * 66 * 4 <= 2 * sizeof(ChunkBuf<T>), "lds");
  const int id = blockIdx.x;
  if (id < n_global_wg) {
    const int per_bh = a.n_split * n_qgroups;
    const int bh = id / per_bh;
    const int rem = id % per_bh;
    global_split<T, NQB>(a, bh, rem / n_qgroups, rem % n_qgroups, smem);
  } else {
    const int n_band = a.B * a.H * n_tiles;
    const int li = xcd_remap(id - n_global_wg, n_band);
    band_tile<T>(a, li / n_tiles, li % n_tiles, (ChunkBuf<T>*)smem);
  }
}

// Merge the split partials of each global row; one wave per (b, h, r), lane = d.
template <typename T>
__global__ __launch_bounds__(256) void global_combine_kernel(AttnArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int nb = a.gcnt[b];
  (void)h;
  const int d = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const T* bias_row = (const T*)a.bias + (size_t)b * a.S;
  for (int r = wave; r < nb; r += 4) {
    const float* p = a.partials + (size_t)bh * a.n_split * a.G * 66 + (size_t)r * 66;
    float M = kNegBig;
    for (int sp = 0; sp < a.n_split; ++sp) M = fmaxf(M, p[(size_t)sp * a.G * 66]);
    float L = 0.0f, O = 0.0f;
    for (int sp = 0; sp < a.n_split; ++sp) {
      const float* q = p + (size_t)sp * a.G * 66;
      const float f = fast_exp2(q[0] - M);
      L += q[1] * f;
      O += q[2 + d] * f;
    }
    const int s = a.gidx[(size_t)b * a.S + r];
    const bool live = Elem<T>::to_f(bias_row[s]) == 0.0f;
    T* dst = (T*)a.out + (size_t)b * a.out_sb + (size_t)h * a.out_sh + (size_t)s * a.out_ss;
    dst[d] = Elem<T>::from_f(live ? O / L : 0.0f);
  }
}

template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  const int n_tiles = (a.S + kTileRows - 1) / kTileRows;
  const int64_t n_band = (int64_t)a.B * a.H * n_tiles;
  const int nqb = a.G <= 32 ? 1 : 2;
  const int n_qgroups = a.G > 0 ? (a.G + 32 * nqb - 1) / (32 * nqb) : 0;
  const int64_t n_global = a.G > 0 ? (int64_t)a.B * a.H * a.n_split * n_qgroups : 0;
  const int64_t grid = n_band + n_global;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.ev_begin) {
    hipError_t e0 = hipEventRecord(a.ev_begin, st);
    if (e0 != hipSuccess) return e0;
  }
  if (nqb == 1)
    attn_mfma_kernel<T, 1><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles, (int)n_global,
                                                                n_qgroups);
  else
    attn_mfma_kernel<T, 2><<<(unsigned)grid, kThreads, 0, st>>>(a, n_tiles, (int)n_global,
                                                                n_qgroups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_end) {
    e = hipEventRecord(a.ev_end, st);
    if (e != hipSuccess) return e;
  }
  if (a.G > 0) {
    global_combine_kernel<T><<<a.B * a.H, 256, 0, st>>>(a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

size_t attn_partials_bytes(int B, int H, int S, int G, int* n_split, int* split_len) {
  // about 512 global workgroups in total, at least 256 keys each
  int64_t len = ((int64_t)B * H * S / 512 + 63) / 64 * 64;
  if (len < 256) len = 256;
  const int64_t s64 = ((int64_t)S + 63) / 64 * 64;
  if (len > s64) len = s64;
  const int ns = (int)((S + len - 1) / len);
  if (n_split) *n_split = ns;
  if (split_len) *split_len = (int)len;
  return (size_t)B * H * ns * (size_t)(G > 0 ? G : 1) * 66 * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 1: return launch_t<f16>(a, st);
    case 2: return launch_t<bf16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lf
