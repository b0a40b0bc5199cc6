// fp32 band + global attention on the vector ALUs (no fp32 matrix path needed at
// the fp32 parity tolerance).
//
// [FT-LF] = the page "FasterTransformer Longformer 推理加速实践", section
// "Longformer Encoder 计算流程", per-layer steps 3-4: local rows normalise over
// their window plus the global tokens, global rows over the whole sequence,
// padded rows are zeroed; the shifted mask is an additive score bias
// (preprocessing item 2).
//
// A workgroup of 4 waves owns 64 query slots of one (batch, head): either local rows
// s0..s0+63 or global rows r0..r0+63; lane l of every wave holds query slot l.  Keys
// stream through LDS in chunks of 64 rows (K and V in fp32, loaded into registers one
// chunk ahead); the chunk's 16 groups of 4 keys go round robin to the waves, and each
// wave runs an online softmax over its groups for all 64 queries: 4 independent dot
// products per group (K rows read as 16-byte broadcasts), scores in log2 units (scaled
// by log2 e, exponentials by the hardware exp2), a running max that moves only when
// passed by 8.  At the end the 4 waves' states (m, l, o) are merged in LDS and the
// merged rows written.  Global keys (positions global_idx[0..n_b)) come first for local
// rows; band keys are [max(n_b, s0 - W/2), min(S-1, s0+63+W/2)] when the global tokens
// lead, or [max(0, s0 - W/2), ...] minus the positions whose global-mask value is zero
// when they may sit anywhere (any_pos).  Global rows with few rows per tile split the
// lanes into key streams, and their keys into the split plan's key splits (one
// workgroup each, states combined by merge_kernel).
#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

namespace {

constexpr int kRows = 64;              // query slots per workgroup
constexpr int kChunk = 64;             // keys per LDS chunk
constexpr int kVw = 4;                 // waves per workgroup
constexpr float kLazy = 8.0f;          // the running max moves only when passed by this
                                       // much (log2 units): p <= 2^8, no overflow in fp32
constexpr int kGrp = 4;                // keys scored together
constexpr int kLd = 68;                // LDS row pitch (floats): 16-byte aligned rows
constexpr int kStP = 36;               // merge state per query: m, l, pad, pad, 32 dims of o
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;    // running-max start: finite, so exp2 never sees inf-inf
static_assert(2 * kChunk * kLd <= kVw * kRows * kStP, "chunk buffers fit in the merge buffer");

// One thread's part of a chunk of key slots 0 .. 63: slot i holds row r = (gather ?
// rows[first + i] : first + i) when i < count and r < S, else zeros; thread t carries
// dims 16 (t % 4) .. + 15 of slot t / 4 of K and V, and (t % 4 == 0) the slot's additive
// bias (the shifted local mask), -inf for an empty slot or (excl_row given) a position
// whose global-mask value is zero, which is not a band key.  Loaded into registers one
// chunk ahead, stored to LDS when the previous chunk is consumed.
struct ChunkRegs {
  f32x4 k[4], v[4];
  float bias;   // the shifted local mask at the row
  float excl;   // its global-mask value (1 when positions are not excluded)
  bool valid;
};

__device__ inline void load_chunk(ChunkRegs& cr, const float* __restrict__ kh,
                                  const float* __restrict__ vh, const int32_t* __restrict__ rows,
                                  int first, int count, int S, bool gather,
                                  const float* __restrict__ bias_row,
                                  const float* __restrict__ excl_row) {
  const int t = threadIdx.x;
  const int i = t >> 2, qd = t & 3;
  int row = -1;
  if (i < count) row = gather ? rows[first + i] : first + i;
  if (row >= S) row = -1;
  cr.valid = row >= 0;
  const size_t off = (size_t)(row < 0 ? 0 : row) * 64 + 16 * qd;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    cr.k[c] = *(const f32x4*)(kh + off + 4 * c);
    cr.v[c] = *(const f32x4*)(vh + off + 4 * c);
  }
  // raw values only: nothing tests a loaded value before the store, so nothing waits
  cr.bias = bias_row[row < 0 ? 0 : row];
  cr.excl = excl_row ? excl_row[row < 0 ? 0 : row] : 1.0f;
}

__device__ inline void store_chunk(const ChunkRegs& cr, float* __restrict__ kl,
                                   float* __restrict__ vl, float* __restrict__ bl) {
  const int t = threadIdx.x;
  const int i = t >> 2, qd = t & 3;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    *(f32x4*)(kl + i * kLd + 16 * qd + 4 * c) = cr.valid ? cr.k[c] : f32x4{};
    *(f32x4*)(vl + i * kLd + 16 * qd + 4 * c) = cr.valid ? cr.v[c] : f32x4{};
  }
  if (qd == 0) bl[i] = cr.valid && cr.excl != 0.0f ? cr.bias : -INFINITY;
}

// Grid: first the global tiles, n_global_tiles x n_gs per (b, h) (tile gt, key split
// sp = the keys [sp split_len, (sp + 1) split_len) of the sequence), then the band tiles,
// n_local_tiles per (b, h).  The short global tiles go first so that they run beside the
// first round of band tiles instead of adding a round at the end.  With n_gs > 1 a
// global tile writes its rows' unnormalised states (m in log2 units, l, o) to the
// partials, which merge_kernel combines.
__global__ __launch_bounds__(64 * kVw) void attn_valu_kernel(AttnArgs a, int n_local_tiles,
                                                             int n_global_tiles, int n_gs) {
  // key chunks while streaming, then (reused) the merge state of half the dims
  __shared__ __attribute__((aligned(16))) float lds[kVw * kRows * kStP];
  __shared__ float bs[kChunk];
  float* ks = lds;
  float* vs = lds + kChunk * kLd;
  float* st = lds;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n_gwg = a.B * a.H * n_global_tiles * n_gs;   // global tiles in the grid
  const bool is_global_tile = (int)blockIdx.x < n_gwg;
  const int per_head = is_global_tile ? n_global_tiles * n_gs : n_local_tiles;
  const int idx = is_global_tile ? blockIdx.x : blockIdx.x - n_gwg;
  const int bh = idx / per_head;
  const int tile = idx % per_head;   // band tile, or gt * n_gs + sp
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int S = a.S;
  const int half = a.W / 2;
  const int nb = a.gcnt[b];
  const size_t head = ((size_t)b * a.H + h) * (size_t)S * 64;
  const float* bias = (const float*)a.bias + (size_t)b * S;
  const int32_t* gidx = a.gidx + (size_t)b * S;
  const int gt = is_global_tile ? tile / n_gs : 0;   // global tile
  const int sp = is_global_tile ? tile % n_gs : 0;   // its key split
  const float* gmask = a.any_pos ? (const float*)a.global_mask + (size_t)b * S : nullptr;

  // A global tile with few rows splits its lanes into key streams: lane = slot q (below
  // P, the rows rounded up to a power of two) + P * stream r, r < R = min(4, 64 / P);
  // stream r takes every R-th group of keys of the wave's part of each chunk.
  int P = kRows, R = 1;
  if (is_global_tile) {
    const int rows = min(kRows, min(nb, a.G) - gt * kRows);
    while (P / 2 >= rows && P > kRows / 4) P /= 2;
    R = kRows / P;
  }
  const int q = lane & (P - 1);    // query slot
  const int rs = lane / P;         // key stream

  int s;            // output position of this lane's query slot
  bool active;      // the slot holds a row this kernel computes
  const float* qrow;
  if (!is_global_tile) {
    const int s0 = tile * kRows;
    s = s0 + lane;
    active = s < S && (gmask ? gmask[s] != 0.0f : s >= nb);
    qrow = (const float*)a.q + head + (size_t)(active ? s : 0) * 64;
  } else {
    const int r = gt * kRows + q;
    active = r < min(nb, a.G);   // (a count above G breaks a precondition: rows past G are not read)
    s = active ? gidx[r] : 0;
    qrow = (const float*)a.qg + (((size_t)b * a.H + h) * a.G + (active ? r : 0)) * 64;
  }
  // the same slots in every wave: the whole workgroup leaves together
  if (__ballot(active) == 0ull) return;

  const float qs = active ? a.scale * kLog2e : 0.0f;   // scores in log2 units
  float qv[64];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const f32x4 x = *(const f32x4*)(qrow + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[4 * c + e] = x[e] * qs;
  }
  float acc[64];
#pragma unroll
  for (int d = 0; d < 64; ++d) acc[d] = 0.0f;
  float m = kNegBig, l = 0.0f;

  // Chunks: the gathered global keys (local rows only), then the contiguous keys (the
  // band of a local tile, the whole sequence for a global tile).
  const int n_gather = is_global_tile ? 0 : (nb + kChunk - 1) / kChunk;
  int lo = 0, hi = S - 1;
  if (is_global_tile && n_gs > 1) {
    lo = sp * a.split_len;
    hi = min(S - 1, lo + a.split_len - 1);
  } else if (!is_global_tile) {
    const int s0 = tile * kRows;
    lo = max(gmask ? 0 : nb, s0 - half);
    hi = min(S - 1, s0 + kRows - 1 + half);
  }
  // Contiguous chunks start at multiples of kChunk (keys below lo are masked), so a key's
  // wave and place in the order of the sums depend on its position alone: whether the
  // global tokens are known to lead (lo = n_b) or are excluded by the global mask
  // (lo = 0) gives bit-identical rows.
  const int base = lo / kChunk * kChunk;   // a global tile's split starts on a chunk
  const int n_chunks = n_gather + (hi >= base ? (hi - base + kChunk) / kChunk : 0);
  const float* kh = (const float*)(is_global_tile ? a.kg : a.k) + head;
  const float* vh = (const float*)(is_global_tile ? a.vg : a.v) + head;
  auto chunk_first = [&](int c) { return c < n_gather ? c * kChunk : base + (c - n_gather) * kChunk; };
  auto chunk_count = [&](int c) {
    return c < n_gather ? min(kChunk, nb - c * kChunk) : min(kChunk, hi - chunk_first(c) + 1);
  };
  auto chunk_load = [&](ChunkRegs& cr, int c) {
    const bool g = c < n_gather;
    load_chunk(cr, kh, vh, gidx, chunk_first(c), chunk_count(c), S, g, bias,
               !g && !is_global_tile ? gmask : nullptr);
  };
  ChunkRegs next;
  if (n_chunks > 0) chunk_load(next, 0);
  for (int c = 0; c < n_chunks; ++c) {
    const bool gather = c < n_gather;
    const int first = chunk_first(c);
    const int cnt = chunk_count(c);
    const bool band = !gather && !is_global_tile;
    __syncthreads();  // the previous chunk is consumed
    store_chunk(next, ks, vs, bs);
    __syncthreads();
    if (c + 1 < n_chunks) chunk_load(next, c + 1);  // in flight while this chunk is consumed
    // this wave's keys of the chunk, kGrp at a time
    // groups of kGrp keys, round robin: wave w, stream rs takes groups w + kVw (rs + R t)
    for (int i0 = kGrp * (w + kVw * rs); i0 < cnt; i0 += kGrp * kVw * R) {
      float sc[kGrp];
#pragma unroll
      for (int k = 0; k < kGrp; ++k) sc[k] = 0.0f;
#pragma unroll
      for (int d4 = 0; d4 < 16; ++d4) {
        // at most 4 x 16 bytes per key in flight: the loads are not all hoisted
        if (d4 % 4 == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kGrp; ++k) {
          const f32x4 k4 = *(const f32x4*)&ks[(i0 + k) * kLd + 4 * d4];
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[k] = fmaf(qv[4 * d4 + e], k4[e], sc[k]);
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < kGrp; ++k) {
        // branch-free: slots past cnt hold bias -inf (bs has kChunk entries)
        const int i = i0 + k;
        const int j = first + i;
        const float bi = bs[i];
        const bool ok = active & (bi != -INFINITY) &
                        (!band | ((j >= lo) & (j - s <= half) & (s - j <= half)));
        sc[k] = ok ? fmaf(bi, kLog2e, sc[k]) : -INFINITY;
        mx = fmaxf(mx, sc[k]);
      }
      if (mx > m + kLazy) {
        const float alpha = __builtin_amdgcn_exp2f(m - mx);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < 64; ++d) acc[d] *= alpha;
        m = mx;
      }
#pragma unroll
      for (int k = 0; k < kGrp; ++k) {
        const float p = sc[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[k] - m);
        l += p;
#pragma unroll
        for (int d4 = 0; d4 < 16; ++d4) {
          if (d4 % 8 == 0) __builtin_amdgcn_sched_barrier(0);
          const f32x4 v4 = *(const f32x4*)&vs[(i0 + k) * kLd + 4 * d4];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * d4 + e] = fmaf(p, v4[e], acc[4 * d4 + e]);
        }
      }
    }
  }

  // merge the states of the 4 waves (and R streams), 32 dims at a time: thread ->
  // (query slot q of stream 0, dims 32 half + 8 w .. + 7)
  const bool live = active && bias[s] == 0.0f;
  float* out = (float*)a.out + (size_t)b * a.out_sb + (size_t)h * a.out_sh + (size_t)s * a.out_ss;
  float* mine = st + (w * kRows + lane) * kStP;
  const int n_st = kVw * R;
#pragma unroll
  for (int hd = 0; hd < 2; ++hd) {
    __syncthreads();  // the chunk buffers (or the previous half) are no longer read
    mine[0] = m;
    mine[1] = l;
#pragma unroll
    for (int d4 = 0; d4 < 8; ++d4) {
      const int d = 32 * hd + 4 * d4;
      *(f32x4*)&mine[4 + 4 * d4] = f32x4{acc[d], acc[d + 1], acc[d + 2], acc[d + 3]};
    }
    __syncthreads();
    if (active && rs == 0) {
      // state u: wave u % 4, stream u / 4
      auto state = [&](int u) { return st + ((u % kVw) * kRows + q + P * (u / kVw)) * kStP; };
      float M = kNegBig;
      for (int u = 0; u < n_st; ++u) M = fmaxf(M, state(u)[0]);
      float L = 0.0f;
      f32x4 o[2] = {};
      for (int u = 0; u < n_st; ++u) {
        const float* su = state(u);
        const float f = __builtin_amdgcn_exp2f(su[0] - M);
        L += su[1] * f;
#pragma unroll
        for (int c = 0; c < 2; ++c) o[c] += *(const f32x4*)&su[4 + 8 * w + 4 * c] * f;
      }
      if (is_global_tile && n_gs > 1) {
        float* part = a.partials +
                      (((size_t)bh * n_gs + sp) * a.G + gt * kRows + q) * kPartPitch;
        if (hd == 0 && w == 0) {
          part[0] = M;
          part[1] = L;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) *(f32x4*)(part + 4 + 32 * hd + 8 * w + 4 * c) = o[c];
      } else {
        const float inv = live ? 1.0f / L : 0.0f;
#pragma unroll
        for (int c = 0; c < 2; ++c)
          *(f32x4*)(out + 32 * hd + 8 * w + 4 * c) = live ? o[c] * inv : f32x4{};
      }
    }
  }
}

// The global rows of split global tiles: row r of (b, h) combines its n_gs (<= 64)
// partial states (o = sum_sp o_sp 2^(m_sp - M), l likewise, M = max_sp m_sp) and is
// written at position global_idx[r] (zero when that position is padding).  One
// workgroup per (b, h); wave w takes rows w, w + 4, ...  Lane j first holds split j's
// m and l (max and sum by butterfly), then lane = dimension, summed over the splits in
// order, 8 splits' loads issued together.
__global__ __launch_bounds__(64 * kVw) void merge_kernel(AttnArgs a, int n_gs) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int nb = min(a.gcnt[b], a.G);
  const float* bias = (const float*)a.bias + (size_t)b * a.S;
  const size_t step = (size_t)a.G * kPartPitch;
  for (int r = w; r < nb; r += kVw) {
    const float* p0 = a.partials + ((size_t)bh * n_gs * a.G + r) * kPartPitch;
    float mj = kNegBig, lj = 0.0f;
    if (lane < n_gs) {
      mj = p0[lane * step];
      lj = p0[lane * step + 1];
    }
    float M = mj;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float fj = lane < n_gs ? __builtin_amdgcn_exp2f(mj - M) : 0.0f;
    float L = fj * lj;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    // 8 splits per round, loads first (indices clamped; lanes past n_gs hold fj = 0)
    float o = 0.0f;
    for (int sp0 = 0; sp0 < n_gs; sp0 += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = p0[min(sp0 + k, n_gs - 1) * step + 4 + lane];
#pragma unroll
      for (int k = 0; k < 8; ++k) o += v[k] * __shfl(fj, sp0 + k);
    }
    const int s = a.gidx[(size_t)b * a.S + r];
    const bool live = bias[s] == 0.0f;
    float* out = (float*)a.out + (size_t)b * a.out_sb + (size_t)h * a.out_sh + (size_t)s * a.out_ss;
    out[lane] = live ? o / L : 0.0f;
  }
}

}  // namespace

hipError_t launch_attention_fp32(const AttnArgs& a, hipStream_t st) {
  if (a.dtype != 0) return hipErrorInvalidValue;
  const int n_local = (a.S + kRows - 1) / kRows;
  const int n_global = (a.G + kRows - 1) / kRows;
  // key splits of the global rows when there is room for their partial states (the
  // split plan's, whose lengths are multiples of the chunk)
  const int n_gs = a.G > 0 && a.partials && a.n_split > 1 && a.n_split <= 64 ? a.n_split : 1;
  const int64_t grid = (int64_t)a.B * a.H * (n_local + n_global * n_gs);
  if (a.ev_begin) {
    hipError_t e0 = hipEventRecord(a.ev_begin, st);
    if (e0 != hipSuccess) return e0;
  }
  attn_valu_kernel<<<(unsigned)grid, 64 * kVw, 0, st>>>(a, n_local, n_global, n_gs);
  if (n_gs > 1) merge_kernel<<<(unsigned)(a.B * a.H), 64 * kVw, 0, st>>>(a, n_gs);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.ev_end) e = hipEventRecord(a.ev_end, st);
  return e;
}

}  // namespace lf
