// C ABI of the library: argument validation (pure host code, runs before any HIP
// call), workspace layout, dispatch to the kernels, status / error text.
//
// [FT-LF] = the page "FasterTransformer Longformer 推理加速实践：PyTorch 集成、输入约束与
// 端到端性能解析".  The shape rules are its four hard constraints (section
// "使用前提：四条硬性约束"); where the page's implementation aborts the process on a
// violation, these entry points return LF_ERR_INVALID_ARGUMENT instead.
#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/lf.h"
#include "lf_internal.h"

namespace {

thread_local std::string g_last_error;

// Kernel timing hook state (per thread).
struct Timing {
  bool on = false;
  int cap = 0;
  int used = 0;
  std::vector<hipEvent_t> begin, end;
};
thread_local Timing g_timing;

void timing_release() {
  for (hipEvent_t e : g_timing.begin) hipEventDestroy(e);
  for (hipEvent_t e : g_timing.end) hipEventDestroy(e);
  g_timing = Timing();
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return LF_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(LF_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t dtype_size(int dtype) { return dtype == LF_F32 ? 4 : 2; }

bool known_dtype(int dtype) { return dtype == LF_F32 || dtype == LF_F16 || dtype == LF_BF16; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Shape rules of the attention entry points; returns LF_OK or an error code.
int validate_attn(int dtype, int B, int H, int S, int W, int G) {
  if (!known_dtype(dtype)) return fail(LF_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (B < 1 || H < 1 || S < 1)
    return fail(LF_ERR_INVALID_ARGUMENT, "B, H, S must be >= 1 (got %d, %d, %d)", B, H, S);
  if (W < 2 || (W & 1))
    return fail(LF_ERR_INVALID_ARGUMENT, "window W must be even and >= 2 (got %d)", W);
  if (S % W != 0)
    return fail(LF_ERR_INVALID_ARGUMENT, "S %% W must be 0 (S=%d, W=%d)", S, W);
  if (S < 2 * W)
    return fail(LF_ERR_INVALID_ARGUMENT, "S must be >= 2*W (S=%d, W=%d)", S, W);
  if (G < 0 || G > W)
    return fail(LF_ERR_INVALID_ARGUMENT, "G must satisfy 0 <= G <= W (G=%d, W=%d)", G, W);
  if ((int64_t)B * H * S > INT_MAX)
    return fail(LF_ERR_INVALID_ARGUMENT, "B*H*S exceeds 2^31-1");
  if (dtype != LF_F32 && (int64_t)S * 128 > INT_MAX)
    return fail(LF_ERR_INVALID_ARGUMENT, "S must be < 2^24 for fp16 / bf16 (got %d)", S);
  return LF_OK;
}

int null_check(const char* names, std::initializer_list<const void*> ptrs) {
  int i = 0;
  for (const void* p : ptrs) {
    if (!p) {
      // names is a comma-separated list in the same order as ptrs
      const char* s = names;
      for (int j = 0; j < i && s; ++j) {
        s = strchr(s, ',');
        if (s) ++s;
      }
      std::string nm = s ? std::string(s, strcspn(s, ",")) : "?";
      return fail(LF_ERR_INVALID_ARGUMENT, "null pointer: %s", nm.c_str());
    }
    ++i;
  }
  return LF_OK;
}

// Attention workspace: [B*H int split tickets][global-row partial states].
struct AttnWs {
  size_t partials_off;  // bytes; the tickets start at offset 0
  size_t total;
  int n_split, split_len;
};

AttnWs attn_ws(int B, int H, int S, int G) {
  AttnWs w;
  lf::attn_split_plan(S, &w.n_split, &w.split_len);
  w.partials_off = align256((size_t)B * H * sizeof(int));
  w.total = w.partials_off + align256((size_t)B * H * w.n_split * (size_t)(G > 0 ? G : 1) *
                                      lf::kPartPitch * sizeof(float));
  return w;
}

lf::AttnArgs make_args(int dtype, const void* q, const void* k, const void* v, const void* qg,
                       const void* kg, const void* vg, const int32_t* gidx, const int32_t* gcnt,
                       const void* bias, int B, int H, int S, int W, int G, void* out,
                       int* tickets, float* partials, const AttnWs& ws) {
  lf::AttnArgs a;
  a.dtype = dtype;
  a.raw = 0;
  a.any_pos = 0;
  a.q = q; a.k = k; a.v = v; a.qg = qg; a.kg = kg; a.vg = vg;
  a.local_mask = nullptr; a.global_mask = nullptr;
  a.gidx = gidx; a.gcnt = gcnt; a.bias = bias; a.out = out;
  a.out_ss = 64;
  a.out_sh = (int64_t)S * 64;
  a.out_sb = (int64_t)H * S * 64;
  a.B = B; a.H = H; a.S = S; a.W = W; a.G = G;
  a.scale = 0.125f;
  a.counters = tickets;
  a.partials = partials;
  a.n_split = ws.n_split;
  a.split_len = ws.split_len;
  a.ev_begin = nullptr;
  a.ev_end = nullptr;
  if (g_timing.on && g_timing.used < g_timing.cap) {
    a.ev_begin = g_timing.begin[g_timing.used];
    a.ev_end = g_timing.end[g_timing.used];
    ++g_timing.used;
  }
  return a;
}

// Shape rules of the encoder layer: the attention rules plus hidden == 64 * H, hidden
// and ffn multiples of 128 (GEMM tiles) and LayerNorm widths the row kernel takes.
int validate_layer(int dtype, int B, int S, int hidden, int H, int ffn, int W, int G) {
  if (!known_dtype(dtype)) return fail(LF_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (int e = validate_attn(dtype, B, H, S, W, G)) return e;
  if (hidden != 64 * H)
    return fail(LF_ERR_INVALID_ARGUMENT, "hidden must be 64*H (hidden=%d, H=%d)", hidden, H);
  if (hidden % 128 != 0 || ffn % 128 != 0 || ffn < 128)
    return fail(LF_ERR_INVALID_ARGUMENT, "hidden and ffn must be multiples of 128 (got %d, %d)",
                hidden, ffn);
  if (!lf::layernorm_width_ok(hidden))
    return fail(LF_ERR_INVALID_ARGUMENT, "hidden must be 256, 512, 768, 1024, 2048 or 4096");
  if (G > S) return fail(LF_ERR_INVALID_ARGUMENT, "G must be <= S");
  const int64_t M = (int64_t)B * S;
  if (M * ffn * (int64_t)dtype_size(dtype) > INT_MAX || M * hidden * 4 > (int64_t)1 << 40)
    return fail(LF_ERR_INVALID_ARGUMENT, "B*S*ffn too large for 32-bit GEMM offsets");
  return LF_OK;
}

// Encoder-layer workspace: the attention tickets and partials first (so the
// tickets sit at offset 0), then q, k, v, kg, vg, qg, the attention output, the
// fp32 pre-LayerNorm buffer, h1 in fp32 and in the layer dtype, and the FFN
// intermediate (which reuses the q..vg area when it fits: they are dead by then).
struct LayerWs {
  size_t act_bytes, qkv_off, qg_off, attn_off, z_off, h1f_off, h1t_off, u_off, part_off, total;
  size_t pidx_off, pcnt_off, pbias_off;   // masks preprocessed inside a layer call (fp32,
                                          // or global tokens anywhere): index, count, bias
  int split_o, split_ffn2;   // split-K factors of the GEMMs with small grids
};

LayerWs layer_ws(int dtype, int B, int S, int hidden, int H, int ffn, int G) {
  LayerWs L;
  const size_t es = dtype_size(dtype), M = (size_t)B * S;
  const AttnWs aw = attn_ws(B, H, S, G);
  size_t off = align256(aw.total);
  L.act_bytes = align256(M * hidden * es);
  L.qkv_off = off; off += 5 * L.act_bytes;
  L.qg_off = off; off += align256((size_t)B * (G > 0 ? G : 1) * hidden * es);
  L.attn_off = off; off += L.act_bytes;
  L.z_off = off; off += align256(M * hidden * 4);
  L.h1f_off = off; off += align256(M * hidden * 4);
  L.h1t_off = off; off += L.act_bytes;
  const size_t u_bytes = align256(M * (size_t)ffn * es);
  if (u_bytes <= 5 * L.act_bytes) {
    L.u_off = L.qkv_off;
  } else {
    L.u_off = off;
    off += u_bytes;
  }
  // fp32 partial sums of the split-K GEMMs (output projection, FFN2), one at a time
  L.split_o = lf::gemm_splits((int)M, hidden, hidden);
  L.split_ffn2 = lf::gemm_splits((int)M, hidden, ffn);
  size_t part = 0;
  if (L.split_o > 1) part = (size_t)L.split_o * M * hidden * 4;
  if (L.split_ffn2 > 1) part = std::max(part, (size_t)L.split_ffn2 * M * hidden * 4);
  L.part_off = off;
  off += align256(part);
  // masks preprocessed inside the call: fp32 attention runs on the vector ALUs from
  // them, and global tokens at any positions need the index
  L.pidx_off = off; off += align256(M * 4);
  L.pcnt_off = off; off += align256((size_t)B * 4);
  L.pbias_off = off; off += align256(M * es);
  L.total = off;
  return L;
}

// Masks of one layer call: raw (read by the attention kernel) or preprocessed; any:
// the global tokens may sit anywhere (the global queries are gathered through the
// index, the attention runs its globals-anywhere mode).
struct LayerMasks {
  bool raw = true;
  bool any = false;
  const void* local_mask = nullptr;
  const void* global_mask = nullptr;
  const int32_t* gidx = nullptr;
  const int32_t* gcnt = nullptr;
  const void* bias = nullptr;
};

int check_layer_call(const lf_layer_weights* w, int G, const void* x, const void* local_mask,
                     const void* global_mask, const void* y, const void* workspace) {
  if (!w) return fail(LF_ERR_INVALID_ARGUMENT, "null pointer: weights");
  if (int e = null_check("x,local_mask,global_mask,y,workspace,w_proj,b_proj,w_o,b_o,ln1_g,"
                         "ln1_b,w_ffn1,b_ffn1,w_ffn2,b_ffn2,ln2_g,ln2_b",
                         {x, local_mask, global_mask, y, workspace, w->w_proj, w->b_proj, w->w_o,
                          w->b_o, w->ln1_g, w->ln1_b, w->w_ffn1, w->b_ffn1, w->w_ffn2, w->b_ffn2,
                          w->ln2_g, w->ln2_b}))
    return e;
  if (G > 0 && (!w->w_qg || !w->b_qg))
    return fail(LF_ERR_INVALID_ARGUMENT, "null pointer: w_qg / b_qg (G > 0)");
  return LF_OK;
}

int check_layer_ws(const void* workspace, size_t ws_bytes, size_t need, float attn_scale,
                   float ln_eps) {
  if (ws_bytes < need)
    return fail(LF_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  if ((uintptr_t)workspace % 256 != 0)
    return fail(LF_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (!(attn_scale > 0.0f) || !(ln_eps > 0.0f))
    return fail(LF_ERR_INVALID_ARGUMENT, "attn_scale and ln_eps must be > 0");
  return LF_OK;
}

// Stack workspace: one layer's workspace (tickets first), then the preprocessed
// masks and one activation buffer for the layer outputs.
struct StackWs {
  LayerWs layer;
  size_t gidx_off, gcnt_off, bias_off, act_off, total;
};

StackWs stack_ws(int dtype, int B, int S, int hidden, int H, int ffn, int G) {
  StackWs W;
  W.layer = layer_ws(dtype, B, S, hidden, H, ffn, G);
  size_t off = W.layer.total;
  W.gidx_off = off; off += align256((size_t)B * S * 4);
  W.gcnt_off = off; off += align256((size_t)B * 4);
  W.bias_off = off; off += align256((size_t)B * S * dtype_size(dtype));
  W.act_off = off; off += W.layer.act_bytes;
  W.total = off;
  return W;
}

// The attention launch of one call: MFMA kernel for fp16 / bf16, vector ALU for fp32.
hipError_t run_attention(const lf::AttnArgs& a, hipStream_t st) {
  return a.dtype == LF_F32 ? lf::launch_attention_fp32(a, st) : lf::launch_attention(a, st);
}

// [FT-LF] per-layer step 6 on two GEMMs: u = GELU(h W1^T + b1) (layer dtype, [M, F]),
// then u W2^T + b2 + resid (fp32) and LayerNorm; FFN2 split over K into `part` when
// its grid is small (the sum happens inside the LayerNorm kernel), else written to
// the fp32 buffer z.  Used by the layer and by lf_ffn_block.
hipError_t run_ffn_two_gemm(int dtype, const void* h, const float* resid, const void* w1,
                            const void* b1, const void* w2, const void* b2, const void* ln_g,
                            const void* ln_b, float ln_eps, int M, int D, int F, int split_ffn2,
                            void* u, float* z, float* part, void* y, hipStream_t st) {
  lf::GemmArgs g;
  memset(&g, 0, sizeof g);
  g.dtype = dtype; g.epi = lf::kEpiGelu;
  g.a = h; g.lda = D;
  g.w = w1; g.ldw = D; g.bias = b1;
  g.M = M; g.N = F; g.K = D;
  g.splits = 1;
  g.out = u; g.ldo = F;
  hipError_t he = lf::launch_gemm(g, st);
  if (he != hipSuccess) return he;
  lf::GemmArgs g2;
  memset(&g2, 0, sizeof g2);
  g2.dtype = dtype;
  g2.a = u; g2.lda = F;
  g2.w = w2; g2.ldw = F; g2.bias = b2;
  g2.M = M; g2.N = D; g2.K = F;
  g2.splits = 1;
  if (split_ffn2 > 1) {
    g2.epi = lf::kEpiPartial;
    g2.splits = split_ffn2;
    g2.part = part;
    if ((he = lf::launch_gemm(g2, st)) != hipSuccess) return he;
    return lf::launch_layernorm_parts(dtype, part, split_ffn2, b2, resid, true, ln_g, ln_b,
                                      ln_eps, M, D, nullptr, y, st);
  }
  g2.epi = lf::kEpiResidF32;
  g2.out = z; g2.ldo = D; g2.resid = resid; g2.ldr = D;
  if ((he = lf::launch_gemm(g2, st)) != hipSuccess) return he;
  return lf::launch_layernorm(dtype, z, ln_g, ln_b, ln_eps, M, D, nullptr, y, st);
}

// One encoder layer ([FT-LF] per-layer steps 1-6) as 7 launches on `st` (8 when the
// masks are preprocessed inside the call); arguments already validated.
int run_layer(int dtype, const lf_layer_weights* w, const void* x, const LayerMasks& mk, int B,
              int S, int hidden, int H, int ffn, int W, int G, float attn_scale, float ln_eps,
              void* y, char* ws, const LayerWs& L, hipStream_t st) {
  const int M = B * S, D = hidden;
  void* qkv[5];
  for (int i = 0; i < 5; ++i) qkv[i] = ws + L.qkv_off + (size_t)i * L.act_bytes;
  void* qg = ws + L.qg_off;
  void* attn = ws + L.attn_off;
  float* z = (float*)(ws + L.z_off);
  float* h1f = (float*)(ws + L.h1f_off);
  void* h1t = ws + L.h1t_off;
  void* u = ws + L.u_off;

  auto gemm = [&](int epi, const void* A, int lda, int a_group, int a_group_stride,
                  const void* Wt, int ldw, const void* bias, int Mr, int N, int K) {
    lf::GemmArgs g;
    memset(&g, 0, sizeof g);
    g.dtype = dtype; g.epi = epi;
    g.a = A; g.lda = lda; g.a_group = a_group; g.a_group_stride = a_group_stride;
    g.w = Wt; g.ldw = ldw; g.bias = bias;
    g.M = Mr; g.N = N; g.K = K;
    g.D = D; g.H = H; g.rows = S;
    g.splits = 1;
    return g;
  };
  float* part = (float*)(ws + L.part_off);
  hipError_t he;
  // masks preprocessed inside this call: fp32 attention reads them, and with global
  // tokens anywhere the global queries and keys go through the index
  const int32_t* gidx = mk.gidx;
  const int32_t* gcnt = mk.gcnt;
  const void* mbias = mk.bias;
  if (mk.raw && (dtype == LF_F32 || mk.any)) {
    int32_t* pidx = (int32_t*)(ws + L.pidx_off);
    int32_t* pcnt = (int32_t*)(ws + L.pcnt_off);
    void* pbias = ws + L.pbias_off;
    if ((he = lf::launch_prep(dtype, mk.global_mask, mk.local_mask, B, S, pidx, pcnt, pbias,
                              nullptr, 0, st)) != hipSuccess)
      return hip_fail(he, "layer mask preprocessing");
    gidx = pidx;
    gcnt = pcnt;
    mbias = pbias;
  }
  // steps 1-2: packed projections split into heads ([B, H, S, 64] each), and the
  // global queries (rows 0 .. G-1 of every sequence, or the rows at the global
  // positions: the first G entries of the index) in the same launch, their few tiles
  // after the projection's
  {
    lf::GemmArgs g = gemm(lf::kEpiHeads, x, D, 0, 0, w->w_proj, D, w->b_proj, M, 5 * D, D);
    for (int i = 0; i < 5; ++i) g.heads[i] = qkv[i];
    if (G > 0) {
      lf::GemmArgs gq = gemm(lf::kEpiHeads, x, D, G, S, w->w_qg, D, w->b_qg, B * G, D, D);
      gq.heads[0] = qg;
      gq.rows = G;
      if (mk.any) gq.a_rows = gidx;
      if ((he = lf::launch_gemm_pair(g, gq, st)) != hipSuccess)
        return hip_fail(he, "projection GEMMs");
    } else if ((he = lf::launch_gemm(g, st)) != hipSuccess) {
      return hip_fail(he, "projection GEMM");
    }
  }
  // steps 3-4: attention, heads joined ([B, S, H * 64])
  {
    AttnWs aw = attn_ws(B, H, S, G);
    lf::AttnArgs a = make_args(dtype, qkv[0], qkv[1], qkv[2], qg, qkv[3], qkv[4], gidx, gcnt,
                               mbias, B, H, S, W, G, attn, (int*)ws,
                               (float*)(ws + aw.partials_off), aw);
    // fp16 / bf16: the MFMA kernel reads the raw masks (leading globals: itself; any
    // positions: with the index); fp32: the vector-ALU kernel reads the preprocessed
    // masks (and the global mask for any positions)
    a.raw = dtype != LF_F32 && (mk.raw || mk.any) ? 1 : 0;
    a.any_pos = mk.any ? 1 : 0;
    a.local_mask = mk.local_mask;
    a.global_mask = mk.global_mask;
    a.out_ss = D;
    a.out_sh = 64;
    a.out_sb = (int64_t)S * D;
    a.scale = attn_scale;
    if ((he = run_attention(a, st)) != hipSuccess) return hip_fail(he, "attention");
  }
  // step 5: output projection + bias + residual (fp32), LayerNorm
  if (L.split_o > 1) {
    // split-K partials, reduced with bias and residual inside the LayerNorm
    lf::GemmArgs g = gemm(lf::kEpiPartial, attn, D, 0, 0, w->w_o, D, w->b_o, M, D, D);
    g.splits = L.split_o;
    g.part = part;
    if ((he = lf::launch_gemm(g, st)) != hipSuccess) return hip_fail(he, "output GEMM");
    if ((he = lf::launch_layernorm_parts(dtype, part, L.split_o, w->b_o, x, false, w->ln1_g,
                                         w->ln1_b, ln_eps, M, D, h1f, h1t, st)) != hipSuccess)
      return hip_fail(he, "LayerNorm 1");
  } else {
    lf::GemmArgs g = gemm(lf::kEpiResidT, attn, D, 0, 0, w->w_o, D, w->b_o, M, D, D);
    g.out = z; g.ldo = D; g.resid = x; g.ldr = D;
    if ((he = lf::launch_gemm(g, st)) != hipSuccess) return hip_fail(he, "output GEMM");
    if ((he = lf::launch_layernorm(dtype, z, w->ln1_g, w->ln1_b, ln_eps, M, D, h1f, h1t, st)) !=
        hipSuccess)
      return hip_fail(he, "LayerNorm 1");
  }
  // step 6: FFN with GELU, second GEMM + bias + residual (fp32), LayerNorm
  if ((he = run_ffn_two_gemm(dtype, h1t, h1f, w->w_ffn1, w->b_ffn1, w->w_ffn2, w->b_ffn2,
                             w->ln2_g, w->ln2_b, ln_eps, M, D, ffn, L.split_ffn2, u, z, part, y,
                             st)) != hipSuccess)
    return hip_fail(he, "FFN");
  return LF_OK;
}

// Scratch of lf_attn_forward / lf_attn_forward_any_globals, per (device, stream).
//  - Split tickets (fp16 / bf16): one slot of kTicketsPerSlot ints of a static device
//    array per (device, stream).  A slot is zero-filled on its stream when it is handed
//    out and every call leaves its tickets zero again, so the calls of one stream,
//    which run in order, share it with no fill.
//  - The rest (global-row partials, the index of the globals-anywhere mode, fp32's
//    preprocessed masks): one device buffer per (device, stream), allocated and, when a
//    call needs more, replaced with stream-ordered hipMallocAsync / hipFreeAsync on that
//    stream, so no call waits for the host.  A per-call allocation and free cost ~2 us
//    per call at the longformer-large shape; the buffer is released by
//    lf_release_stream_scratch or at process end.
// A call holds the lock from the lookup until its kernels are enqueued: a concurrent
// call on the same stream that replaces the buffer enqueues its free after them.
// Streams being captured into a graph get neither: their calls bring their own
// stream-ordered scratch and zero-filled tickets (capture-safe), freed in the graph.
constexpr int kTicketSlots = 64;
constexpr int kTicketsPerSlot = 8192;
static __device__ __align__(256) int g_stream_tickets[kTicketSlots * kTicketsPerSlot];

struct StreamScratch {
  int* tickets = nullptr;   // the stream's ticket slot (nullptr: none left)
  char* buf = nullptr;      // cached scratch buffer
  size_t bytes = 0;
};
struct DeviceScratch {
  int* base = nullptr;      // device address of g_stream_tickets on that device
  int slots_used = 0;
  std::map<hipStream_t, StreamScratch> streams;
};
std::mutex g_scratch_mu;
std::map<int, DeviceScratch> g_scratch;

// The (device, stream) entry, its ticket slot assigned (and zero-filled on st) on first
// use; call with g_scratch_mu held.
int stream_entry(hipStream_t st, StreamScratch** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  DeviceScratch& D = g_scratch[dev];
  if (!D.base) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_stream_tickets));
    if (e != hipSuccess) return hip_fail(e, "ticket slots (hipGetSymbolAddress)");
    D.base = (int*)p;
  }
  auto it = D.streams.find(st);
  if (it == D.streams.end()) {
    StreamScratch ss;
    if (D.slots_used < kTicketSlots) {
      int* p = D.base + (size_t)D.slots_used * kTicketsPerSlot;
      e = lf::launch_fill_i32(p, kTicketsPerSlot, 0, st);
      if (e != hipSuccess) return hip_fail(e, "ticket slot zero-fill");
      ++D.slots_used;
      ss.tickets = p;
    }
    it = D.streams.emplace(st, ss).first;
  }
  *out = &it->second;
  return LF_OK;
}

bool debug_check_enabled() {
  const char* e = getenv("LF_DEBUG_CHECK");
  return e && e[0] == '1';
}

}  // namespace

extern "C" {

const char* lf_status_string(int status) {
  switch (status) {
    case LF_OK: return "ok";
    case LF_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LF_ERR_UNSUPPORTED: return "unsupported";
    case LF_ERR_HIP: return "HIP error";
    case LF_ERR_PRECONDITION: return "precondition violated";
  }
  return "unknown status";
}

const char* lf_last_error(void) { return g_last_error.c_str(); }

int lf_init_global_idx(int dtype, const void* global_mask, int B, int S, int32_t* global_idx,
                       int32_t* global_count, void* stream) {
  if (!known_dtype(dtype)) return fail(LF_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (B < 1 || S < 1) return fail(LF_ERR_INVALID_ARGUMENT, "B, S must be >= 1");
  if ((int64_t)B * S > INT_MAX) return fail(LF_ERR_INVALID_ARGUMENT, "B*S exceeds 2^31-1");
  if (int e = null_check("global_mask,global_idx,global_count",
                         {global_mask, global_idx, global_count}))
    return e;
  hipError_t he = lf::launch_prep(dtype, global_mask, nullptr, B, S, global_idx, global_count,
                                  nullptr, nullptr, 0, (hipStream_t)stream);
  if (he != hipSuccess) return hip_fail(he, "lf_init_global_idx");
  return ok();
}

int lf_mask_shift(int dtype, const void* local_mask, int B, int S, void* local_bias,
                  void* stream) {
  if (!known_dtype(dtype)) return fail(LF_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (B < 1 || S < 1) return fail(LF_ERR_INVALID_ARGUMENT, "B, S must be >= 1");
  if (int e = null_check("local_mask,local_bias", {local_mask, local_bias})) return e;
  hipError_t he = lf::launch_mask_shift(dtype, local_mask, (int64_t)B * S, local_bias,
                                        (hipStream_t)stream);
  if (he != hipSuccess) return hip_fail(he, "lf_mask_shift");
  return ok();
}

size_t lf_attn_workspace_bytes(int dtype, int B, int H, int S, int W, int G) {
  if (validate_attn(dtype, B, H, S, W, G) != LF_OK) return 0;
  return attn_ws(B, H, S, G).total;
}

int lf_attn_forward_pre(int dtype, const void* q, const void* k, const void* v, const void* qg,
                        const void* kg, const void* vg, const int32_t* global_idx,
                        const int32_t* global_count, const void* local_bias, int B, int H, int S,
                        int W, int G, void* out, void* workspace, size_t ws_bytes,
                        void* stream) {
  if (int e = validate_attn(dtype, B, H, S, W, G)) return e;
  if (int e = null_check("q,k,v,kg,vg,global_idx,global_count,local_bias,out,workspace",
                         {q, k, v, kg, vg, global_idx, global_count, local_bias, out, workspace}))
    return e;
  if (G > 0 && !qg) return fail(LF_ERR_INVALID_ARGUMENT, "null pointer: qg (G > 0)");
  const AttnWs ws = attn_ws(B, H, S, G);
  if (ws_bytes < ws.total)
    return fail(LF_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu", ws_bytes, ws.total);
  if (((uintptr_t)workspace) & 255)
    return fail(LF_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  lf::AttnArgs a = make_args(dtype, q, k, v, qg, kg, vg, global_idx, global_count, local_bias, B,
                             H, S, W, G, out, (int*)workspace,
                             (float*)((char*)workspace + ws.partials_off), ws);
  hipError_t he = run_attention(a, (hipStream_t)stream);
  if (he != hipSuccess) return hip_fail(he, "lf_attn_forward_pre");
  return ok();
}

}  // extern "C"

namespace {

// Scratch of one lf_attn_forward-family call, as offsets into one region.  fp16 /
// bf16: [tickets (with_tickets)][global-row partials (G > 0)][index, count (any_pos)];
// fp32: [index][count][shifted mask] (the vector-ALU kernel reads preprocessed masks)
// [global-row partials (G > 0; combined by a second launch, no tickets)].
struct AttnScratch {
  size_t tickets_off, partials_off, idx_off, cnt_off, bias_off, total;
};

AttnScratch attn_scratch(int dtype, int B, int H, int S, int G, bool any_pos, bool with_tickets) {
  AttnScratch c;
  size_t off = 0;
  const size_t n_bs = (size_t)B * S;
  c.tickets_off = c.partials_off = c.idx_off = c.cnt_off = c.bias_off = 0;
  if (dtype == LF_F32) {
    c.idx_off = off; off += align256(n_bs * sizeof(int32_t));
    c.cnt_off = off; off += align256((size_t)B * sizeof(int32_t));
    c.bias_off = off; off += align256(n_bs * dtype_size(dtype));
    if (G > 0) {
      const AttnWs w = attn_ws(B, H, S, G);
      c.partials_off = off;
      off += w.total - w.partials_off;
    }
    c.total = off;
    return c;
  }
  if (with_tickets && G > 0) {
    c.tickets_off = off;
    off += align256((size_t)B * H * sizeof(int));
  }
  if (G > 0) {
    const AttnWs w = attn_ws(B, H, S, G);
    c.partials_off = off;
    off += w.total - w.partials_off;
  }
  if (any_pos) {
    c.idx_off = off; off += align256(n_bs * sizeof(int32_t));
    c.cnt_off = off; off += align256((size_t)B * sizeof(int32_t));
  }
  c.total = off;
  return c;
}

// The launches of lf_attn_forward (any_pos = false) / lf_attn_forward_any_globals
// (any_pos = true) into a given scratch region (layout sc) with given split tickets
// (zero on entry, left zero; fp16 / bf16 with G > 0 only).  fp16 / bf16, leading
// globals: one launch, the kernel reads both masks itself (count of the leading global
// tokens, live-key test of the local mask); globals anywhere: the index partition
// first, then the kernel, which gathers the global keys through it.  fp32: the
// preprocessing kernel, then the vector-ALU kernel.
hipError_t run_attn_forward(int dtype, const void* q, const void* k, const void* v,
                            const void* qg, const void* kg, const void* vg,
                            const void* local_mask, const void* global_mask, int B, int H, int S,
                            int W, int G, void* out, hipStream_t st, bool any_pos, char* scratch,
                            const AttnScratch& sc, const AttnWs& ws, int* tickets) {
  int32_t* gidx = nullptr;
  int32_t* gcnt = nullptr;
  void* bias = nullptr;
  float* partials = nullptr;
  if (dtype == LF_F32) {
    gidx = (int32_t*)(scratch + sc.idx_off);
    gcnt = (int32_t*)(scratch + sc.cnt_off);
    bias = scratch + sc.bias_off;
    hipError_t he = lf::launch_prep(dtype, global_mask, local_mask, B, S, gidx, gcnt, bias,
                                    nullptr, 0, st);
    if (he != hipSuccess) return he;
    if (G > 0) partials = (float*)(scratch + sc.partials_off);
    lf::AttnArgs a = make_args(dtype, q, k, v, qg, kg, vg, gidx, gcnt, bias, B, H, S, W, G, out,
                               nullptr, partials, ws);
    a.any_pos = any_pos ? 1 : 0;
    a.global_mask = global_mask;
    return run_attention(a, st);
  }
  if (G > 0) partials = (float*)(scratch + sc.partials_off);
  if (any_pos) {
    gidx = (int32_t*)(scratch + sc.idx_off);
    gcnt = (int32_t*)(scratch + sc.cnt_off);
    hipError_t he = lf::launch_prep(dtype, global_mask, nullptr, B, S, gidx, gcnt, nullptr,
                                    nullptr, 0, st);
    if (he != hipSuccess) return he;
  }
  lf::AttnArgs a = make_args(dtype, q, k, v, qg, kg, vg, gidx, gcnt, nullptr, B, H, S, W, G, out,
                             tickets, partials, ws);
  a.raw = 1;
  a.any_pos = any_pos ? 1 : 0;
  a.local_mask = local_mask;
  a.global_mask = global_mask;
  return run_attention(a, st);
}

// The mask precondition check; leading: the global tokens must also be contiguous at
// the head of the sequence (lf_attn_forward), not when they may sit anywhere.
int check_masks_impl(int dtype, const void* local_mask, const void* global_mask, int B, int S,
                     int G, void* stream, bool leading) {
  if (!known_dtype(dtype)) return fail(LF_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (B < 1 || S < 1 || G < 0) return fail(LF_ERR_INVALID_ARGUMENT, "bad B, S or G");
  if ((int64_t)B * S >= INT_MAX) return fail(LF_ERR_INVALID_ARGUMENT, "B*S too large");
  if (int e = null_check("local_mask,global_mask", {local_mask, global_mask})) return e;
  hipStream_t st = (hipStream_t)stream;
  int* dflags = nullptr;
  hipError_t he = hipMallocAsync((void**)&dflags, 4 * sizeof(int), st);
  if (he != hipSuccess) return hip_fail(he, "lf_check_masks alloc");
  const int init[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
  int flags[4];
  he = hipMemcpyAsync(dflags, init, sizeof init, hipMemcpyHostToDevice, st);
  if (he == hipSuccess)
    he = lf::launch_check_masks(dtype, local_mask, global_mask, B, S, G, dflags, st);
  if (he == hipSuccess)
    he = hipMemcpyAsync(flags, dflags, sizeof flags, hipMemcpyDeviceToHost, st);
  hipError_t he2 = hipFreeAsync(dflags, st);
  if (he == hipSuccess) he = he2;
  if (he == hipSuccess) he = hipStreamSynchronize(st);
  if (he != hipSuccess) return hip_fail(he, "lf_check_masks");
  if (flags[0] != INT_MAX)
    return fail(LF_ERR_PRECONDITION, "local_mask[%d] is neither 0 nor 1", flags[0] - 1);
  if (flags[1] != INT_MAX)
    return fail(LF_ERR_PRECONDITION, "global_mask[%d] is neither 0 nor -10000", flags[1] - 1);
  if (leading && flags[2] != INT_MAX)
    return fail(LF_ERR_PRECONDITION,
                "global tokens of batch row %d are not contiguous at the sequence head",
                flags[2] - 1);
  if (flags[3] != INT_MAX)
    return fail(LF_ERR_PRECONDITION, "batch row %d has more than G=%d global tokens",
                flags[3] - 1, G);
  return ok();
}

// lf_attn_forward (any_pos = false: the global tokens lead) and
// lf_attn_forward_any_globals (any_pos = true).
int attn_forward_impl(int dtype, const void* q, const void* k, const void* v, const void* qg,
                      const void* kg, const void* vg, const void* local_mask,
                      const void* global_mask, int B, int H, int S, int W, int G, void* out,
                      void* stream, bool any_pos) {
  if (int e = validate_attn(dtype, B, H, S, W, G)) return e;
  if (int e = null_check("q,k,v,kg,vg,local_mask,global_mask,out",
                         {q, k, v, kg, vg, local_mask, global_mask, out}))
    return e;
  if (G > 0 && !qg) return fail(LF_ERR_INVALID_ARGUMENT, "null pointer: qg (G > 0)");
  hipStream_t st = (hipStream_t)stream;
  if (debug_check_enabled()) {
    if (int e = check_masks_impl(dtype, local_mask, global_mask, B, S, G, stream, !any_pos))
      return e;
  }
  const AttnWs ws = attn_ws(B, H, S, G);
  const bool need_tickets = dtype != LF_F32 && G > 0;
  const char* who = any_pos ? "lf_attn_forward_any_globals" : "lf_attn_forward";
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t he = hipStreamIsCapturing(st, &cap);
  if (he != hipSuccess) return hip_fail(he, "hipStreamIsCapturing");
  if (cap != hipStreamCaptureStatusNone) {
    // under capture: scratch and zero-filled tickets of this call alone
    const AttnScratch sc = attn_scratch(dtype, B, H, S, G, any_pos, true);
    char* scratch = nullptr;
    if (sc.total > 0 && (he = hipMallocAsync((void**)&scratch, sc.total, st)) != hipSuccess)
      return hip_fail(he, "attention scratch (hipMallocAsync)");
    int* tickets = need_tickets ? (int*)(scratch + sc.tickets_off) : nullptr;
    if (need_tickets) he = lf::launch_fill_i32(tickets, (int64_t)B * H, 0, st);
    if (he == hipSuccess)
      he = run_attn_forward(dtype, q, k, v, qg, kg, vg, local_mask, global_mask, B, H, S, W, G,
                            out, st, any_pos, scratch, sc, ws, tickets);
    const hipError_t he2 = scratch ? hipFreeAsync(scratch, st) : hipSuccess;
    if (he != hipSuccess) return hip_fail(he, who);
    if (he2 != hipSuccess) return hip_fail(he2, "attention scratch (hipFreeAsync)");
    return ok();
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  StreamScratch* ss = nullptr;
  if (int e = stream_entry(st, &ss)) return e;
  // the stream's ticket slot when it has one and it is large enough, else tickets in
  // the scratch buffer (zero-filled by this call)
  const bool slot = need_tickets && ss->tickets && (int64_t)B * H <= kTicketsPerSlot;
  const AttnScratch sc = attn_scratch(dtype, B, H, S, G, any_pos, need_tickets && !slot);
  if (sc.total > ss->bytes) {
    if (ss->buf && (he = hipFreeAsync(ss->buf, st)) != hipSuccess)
      return hip_fail(he, "attention scratch (hipFreeAsync)");
    ss->buf = nullptr;
    ss->bytes = 0;
    if ((he = hipMallocAsync((void**)&ss->buf, sc.total, st)) != hipSuccess)
      return hip_fail(he, "attention scratch (hipMallocAsync)");
    ss->bytes = sc.total;
  }
  int* tickets = nullptr;
  if (slot) {
    tickets = ss->tickets;
  } else if (need_tickets) {
    tickets = (int*)(ss->buf + sc.tickets_off);
    if ((he = lf::launch_fill_i32(tickets, (int64_t)B * H, 0, st)) != hipSuccess)
      return hip_fail(he, who);
  }
  he = run_attn_forward(dtype, q, k, v, qg, kg, vg, local_mask, global_mask, B, H, S, W, G, out,
                        st, any_pos, ss->buf, sc, ws, tickets);
  if (he != hipSuccess) return hip_fail(he, who);
  return ok();
}

}  // namespace

namespace lf {

size_t attn_forward_scratch_bytes(int dtype, int B, int H, int S, int G) {
  return attn_scratch(dtype, B, H, S, G, false, false).total;
}

int attn_forward_validate(int dtype, const void* q, const void* k, const void* v,
                          const void* qg, const void* kg, const void* vg, const void* local_mask,
                          const void* global_mask, int B, int H, int S, int W, int G,
                          const void* out, size_t scratch_bytes, int ticket_capacity,
                          const char* who) {
  if (int e = validate_attn(dtype, B, H, S, W, G)) return e;
  if (int e = null_check("q,k,v,kg,vg,local_mask,global_mask,out",
                         {q, k, v, kg, vg, local_mask, global_mask, out}))
    return e;
  if (G > 0 && !qg) return fail(LF_ERR_INVALID_ARGUMENT, "null pointer: qg (G > 0)");
  const size_t need = attn_scratch(dtype, B, H, S, G, false, false).total;
  if (need > scratch_bytes)
    return fail(LF_ERR_UNSUPPORTED, "%s: this shape needs %zu bytes of scratch, more than the %zu "
                "available", who, need, scratch_bytes);
  if (dtype != LF_F32 && G > 0 && (int64_t)B * H > ticket_capacity)
    return fail(LF_ERR_UNSUPPORTED, "%s: B*H = %lld exceeds the %d split tickets available", who,
                (long long)B * H, ticket_capacity);
  return LF_OK;
}

int attn_forward_in(int dtype, const void* q, const void* k, const void* v, const void* qg,
                    const void* kg, const void* vg, const void* local_mask,
                    const void* global_mask, int B, int H, int S, int W, int G, void* out,
                    void* stream, char* scratch, size_t scratch_bytes, int* tickets,
                    int ticket_capacity, const char* who) {
  if (int e = attn_forward_validate(dtype, q, k, v, qg, kg, vg, local_mask, global_mask, B, H, S,
                                    W, G, out, scratch_bytes, ticket_capacity, who))
    return e;
  hipStream_t st = (hipStream_t)stream;
  if (debug_check_enabled()) {
    if (int e = check_masks_impl(dtype, local_mask, global_mask, B, S, G, stream, true)) return e;
  }
  const AttnScratch sc = attn_scratch(dtype, B, H, S, G, false, false);
  const hipError_t he = run_attn_forward(dtype, q, k, v, qg, kg, vg, local_mask, global_mask, B,
                                         H, S, W, G, out, st, false, scratch, sc,
                                         attn_ws(B, H, S, G), tickets);
  if (he != hipSuccess) return hip_fail(he, who);
  return ok();
}

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

}  // namespace lf

extern "C" {

int lf_check_masks(int dtype, const void* local_mask, const void* global_mask, int B, int S,
                   int G, void* stream) {
  return check_masks_impl(dtype, local_mask, global_mask, B, S, G, stream, true);
}

int lf_attn_forward(int dtype, const void* q, const void* k, const void* v, const void* qg,
                    const void* kg, const void* vg, const void* local_mask,
                    const void* global_mask, int B, int H, int S, int W, int G, void* out,
                    void* stream) {
  return attn_forward_impl(dtype, q, k, v, qg, kg, vg, local_mask, global_mask, B, H, S, W, G,
                           out, stream, false);
}

int lf_attn_forward_any_globals(int dtype, const void* q, const void* k, const void* v,
                                const void* qg, const void* kg, const void* vg,
                                const void* local_mask, const void* global_mask, int B, int H,
                                int S, int W, int G, void* out, void* stream) {
  return attn_forward_impl(dtype, q, k, v, qg, kg, vg, local_mask, global_mask, B, H, S, W, G,
                           out, stream, true);
}

int lf_release_stream_scratch(void* stream) {
  hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto d = g_scratch.find(dev);
  if (d == g_scratch.end()) return ok();
  auto it = d->second.streams.find(st);
  if (it == d->second.streams.end() || !it->second.buf) return ok();
  e = hipFreeAsync(it->second.buf, st);
  it->second.buf = nullptr;
  it->second.bytes = 0;
  if (e != hipSuccess) return hip_fail(e, "lf_release_stream_scratch");
  return ok();
}

int lf_kernel_timing_start(int capacity) {
  if (capacity < 1 || capacity > 1000000)
    return fail(LF_ERR_INVALID_ARGUMENT, "timing capacity must be in 1..1000000");
  timing_release();
  g_timing.begin.resize(capacity, nullptr);
  g_timing.end.resize(capacity, nullptr);
  for (int i = 0; i < capacity; ++i) {
    hipError_t e = hipEventCreate(&g_timing.begin[i]);
    if (e == hipSuccess) e = hipEventCreate(&g_timing.end[i]);
    if (e != hipSuccess) {
      timing_release();
      return hip_fail(e, "lf_kernel_timing_start");
    }
  }
  g_timing.cap = capacity;
  g_timing.on = true;
  return ok();
}

int lf_kernel_timing_stop(int* launches, double* total_ms) {
  if (!launches || !total_ms) return fail(LF_ERR_INVALID_ARGUMENT, "null output pointer");
  double sum = 0.0;
  const int n = g_timing.used;
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipEventSynchronize(g_timing.end[i]);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timing.begin[i], g_timing.end[i]);
    if (e != hipSuccess) {
      timing_release();
      return hip_fail(e, "lf_kernel_timing_stop");
    }
    sum += ms;
  }
  timing_release();
  *launches = n;
  *total_ms = sum;
  return ok();
}

size_t lf_encoder_layer_workspace_bytes(int dtype, int B, int S, int hidden, int H, int ffn,
                                        int W, int G) {
  if (validate_layer(dtype, B, S, hidden, H, ffn, W, G) != LF_OK) return 0;
  return layer_ws(dtype, B, S, hidden, H, ffn, G).total;
}

}  // extern "C"

namespace {

// lf_encoder_layer (any_pos = false) and lf_encoder_layer_any_globals (true).
int encoder_layer_impl(int dtype, const lf_layer_weights* w, const void* x,
                       const void* local_mask, const void* global_mask, int B, int S, int hidden,
                       int H, int ffn, int W, int G, float attn_scale, float ln_eps, void* y,
                       void* workspace, size_t ws_bytes, void* stream, bool any_pos) {
  if (int e = validate_layer(dtype, B, S, hidden, H, ffn, W, G)) return e;
  if (int e = check_layer_call(w, G, x, local_mask, global_mask, y, workspace)) return e;
  const LayerWs L = layer_ws(dtype, B, S, hidden, H, ffn, G);
  if (int e = check_layer_ws(workspace, ws_bytes, L.total, attn_scale, ln_eps)) return e;
  LayerMasks mk;
  mk.raw = true;
  mk.any = any_pos;
  mk.local_mask = local_mask;
  mk.global_mask = global_mask;
  return run_layer(dtype, w, x, mk, B, S, hidden, H, ffn, W, G, attn_scale, ln_eps, y,
                   (char*)workspace, L, (hipStream_t)stream);
}


// lf_encoder_forward (any_pos = false) and lf_encoder_forward_any_globals (true).
int encoder_forward_impl(int dtype, const lf_layer_weights* w, int n_layers, const void* x,
                         const void* local_mask, const void* global_mask, int B, int S,
                         int hidden, int H, int ffn, int W, int G, float attn_scale, float ln_eps,
                         void* y, void* workspace, size_t ws_bytes, void* stream, bool any_pos) {
  if (int e = validate_layer(dtype, B, S, hidden, H, ffn, W, G)) return e;
  if (n_layers < 1) return fail(LF_ERR_INVALID_ARGUMENT, "n_layers must be >= 1 (got %d)", n_layers);
  if (!w) return fail(LF_ERR_INVALID_ARGUMENT, "null pointer: weights");
  for (int l = 0; l < n_layers; ++l)
    if (int e = check_layer_call(&w[l], G, x, local_mask, global_mask, y, workspace)) return e;
  const StackWs SW = stack_ws(dtype, B, S, hidden, H, ffn, G);
  if (int e = check_layer_ws(workspace, ws_bytes, SW.total, attn_scale, ln_eps)) return e;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  // preprocessing once for every layer ([FT-LF] computation flow: the global-token
  // index and the local-mask shift are computed before the layer loop)
  int32_t* gidx = (int32_t*)(ws + SW.gidx_off);
  int32_t* gcnt = (int32_t*)(ws + SW.gcnt_off);
  LayerMasks mk;
  mk.raw = false;
  mk.any = any_pos;
  mk.local_mask = local_mask;
  mk.global_mask = global_mask;
  mk.gidx = gidx;
  mk.gcnt = gcnt;
  mk.bias = ws + SW.bias_off;
  hipError_t he = lf::launch_prep(dtype, global_mask, local_mask, B, S, gidx, gcnt,
                                  ws + SW.bias_off, nullptr, 0, st);
  if (he != hipSuccess) return hip_fail(he, "preprocessing");
  // the layer outputs alternate between y and one activation buffer, so that the
  // last layer writes y and x is never written
  void* act = ws + SW.act_off;
  const void* in = x;
  for (int l = 0; l < n_layers; ++l) {
    void* out = ((n_layers - 1 - l) % 2 == 0) ? y : act;
    if (int e = run_layer(dtype, &w[l], in, mk, B, S, hidden, H, ffn, W, G, attn_scale, ln_eps,
                          out, ws, SW.layer, st))
      return e;
    in = out;
  }
  return ok();
}

}  // namespace

extern "C" {

size_t lf_encoder_forward_workspace_bytes(int dtype, int B, int S, int hidden, int H, int ffn,
                                          int W, int G) {
  if (validate_layer(dtype, B, S, hidden, H, ffn, W, G) != LF_OK) return 0;
  return stack_ws(dtype, B, S, hidden, H, ffn, G).total;
}

int lf_encoder_layer(int dtype, const lf_layer_weights* w, const void* x, const void* local_mask,
                     const void* global_mask, int B, int S, int hidden, int H, int ffn, int W,
                     int G, float attn_scale, float ln_eps, void* y, void* workspace,
                     size_t ws_bytes, void* stream) {
  return encoder_layer_impl(dtype, w, x, local_mask, global_mask, B, S, hidden, H, ffn, W, G,
                            attn_scale, ln_eps, y, workspace, ws_bytes, stream, false);
}

int lf_encoder_layer_any_globals(int dtype, const lf_layer_weights* w, const void* x,
                                 const void* local_mask, const void* global_mask, int B, int S,
                                 int hidden, int H, int ffn, int W, int G, float attn_scale,
                                 float ln_eps, void* y, void* workspace, size_t ws_bytes,
                                 void* stream) {
  return encoder_layer_impl(dtype, w, x, local_mask, global_mask, B, S, hidden, H, ffn, W, G,
                            attn_scale, ln_eps, y, workspace, ws_bytes, stream, true);
}

int lf_encoder_forward(int dtype, const lf_layer_weights* w, int n_layers, const void* x,
                       const void* local_mask, const void* global_mask, int B, int S, int hidden,
                       int H, int ffn, int W, int G, float attn_scale, float ln_eps, void* y,
                       void* workspace, size_t ws_bytes, void* stream) {
  return encoder_forward_impl(dtype, w, n_layers, x, local_mask, global_mask, B, S, hidden, H,
                              ffn, W, G, attn_scale, ln_eps, y, workspace, ws_bytes, stream,
                              false);
}

int lf_encoder_forward_any_globals(int dtype, const lf_layer_weights* w, int n_layers,
                                   const void* x, const void* local_mask, const void* global_mask,
                                   int B, int S, int hidden, int H, int ffn, int W, int G,
                                   float attn_scale, float ln_eps, void* y, void* workspace,
                                   size_t ws_bytes, void* stream) {
  return encoder_forward_impl(dtype, w, n_layers, x, local_mask, global_mask, B, S, hidden, H,
                              ffn, W, G, attn_scale, ln_eps, y, workspace, ws_bytes, stream,
                              true);
}

}  // extern "C"

// ---------------------------------------------------------------- FFN block
namespace {

// FFN-block workspace.  Two GEMMs: the intermediate u [M, F] in the layer dtype, then
// the fp32 split-K partials of FFN2 or the fp32 pre-LayerNorm rows.  Fused: the fp32
// partials of the F slices only.
struct FfnWs {
  int split;   // FFN2 split-K factor (two GEMMs) or F slices (fused)
  size_t u_off, z_off, total;
};

FfnWs ffn_ws(int dtype, int M, int D, int F, bool fused) {
  FfnWs W;
  const size_t es = dtype_size(dtype);
  if (fused) {
    W.split = lf::ffn_fused_splits(M, F);
    W.u_off = 0;
    W.z_off = 0;
    W.total = align256((size_t)W.split * M * D * 4);
    return W;
  }
  W.split = lf::gemm_splits(M, D, F);
  W.u_off = 0;
  W.z_off = align256((size_t)M * F * es);
  W.total = W.z_off + align256((size_t)std::max(W.split, 1) * M * D * 4);
  return W;
}

int validate_ffn(int dtype, int M, int D, int F, int fused) {
  if (!known_dtype(dtype)) return fail(LF_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (M <= 0) return fail(LF_ERR_INVALID_ARGUMENT, "M must be > 0 (got %d)", M);
  if (D % 128 != 0 || F % 128 != 0 || F < 128)
    return fail(LF_ERR_INVALID_ARGUMENT, "D and F must be multiples of 128 (got %d, %d)", D, F);
  if (!lf::layernorm_width_ok(D))
    return fail(LF_ERR_INVALID_ARGUMENT, "D must be 256, 512, 768, 1024, 2048 or 4096");
  if ((int64_t)M * F * (int64_t)dtype_size(dtype) > INT_MAX ||
      (int64_t)M * D * 4 * 16 > (int64_t)1 << 40)
    return fail(LF_ERR_INVALID_ARGUMENT, "M*F too large for 32-bit GEMM offsets");
  if (fused) {
    if (dtype == LF_F32) return fail(LF_ERR_UNSUPPORTED, "fused FFN: fp16 / bf16 only");
    if (D > 1024 || D % 256 != 0)
      return fail(LF_ERR_UNSUPPORTED, "fused FFN: D must be 256, 512, 768 or 1024 (got %d)", D);
    const int sp = lf::ffn_fused_splits(M, F);
    if (!lf::ffn_fused_ok(dtype, D, F, sp))
      return fail(LF_ERR_UNSUPPORTED, "fused FFN: F must be a multiple of %d (got %d)", 32 * sp, F);
  }
  return LF_OK;
}

}  // namespace

extern "C" {

size_t lf_ffn_block_workspace_bytes(int dtype, int M, int D, int F, int fused) {
  if (validate_ffn(dtype, M, D, F, fused) != LF_OK) return 0;
  return ffn_ws(dtype, M, D, F, fused != 0).total;
}

int lf_ffn_block(int dtype, const void* h, const float* resid, const void* w1, const void* b1,
                 const void* w2, const void* b2, const void* ln_g, const void* ln_b, int M,
                 int D, int F, float ln_eps, int fused, void* y, void* workspace,
                 size_t ws_bytes, void* stream) {
  if (int e = validate_ffn(dtype, M, D, F, fused)) return e;
  if (int e = null_check("h,resid,w1,b1,w2,b2,ln_g,ln_b,y,workspace",
                         {h, resid, w1, b1, w2, b2, ln_g, ln_b, y, workspace}))
    return e;
  const FfnWs W = ffn_ws(dtype, M, D, F, fused != 0);
  if (ws_bytes < W.total)
    return fail(LF_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu bytes", ws_bytes, W.total);
  if ((uintptr_t)workspace % 256 != 0)
    return fail(LF_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (!(ln_eps > 0.0f)) return fail(LF_ERR_INVALID_ARGUMENT, "ln_eps must be > 0");
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t he;
  if (fused) {
    float* part = (float*)ws;
    if ((he = lf::launch_ffn_fused(dtype, h, w1, b1, w2, M, D, F, W.split, part, st)) !=
        hipSuccess)
      return hip_fail(he, "fused FFN");
    if ((he = lf::launch_layernorm_parts(dtype, part, W.split, b2, resid, true, ln_g, ln_b,
                                         ln_eps, M, D, nullptr, y, st)) != hipSuccess)
      return hip_fail(he, "fused FFN LayerNorm");
    return LF_OK;
  }
  float* zp = (float*)(ws + W.z_off);
  if ((he = run_ffn_two_gemm(dtype, h, resid, w1, b1, w2, b2, ln_g, ln_b, ln_eps, M, D, F,
                             W.split, ws + W.u_off, zp, zp, y, st)) != hipSuccess)
    return hip_fail(he, "FFN");
  return LF_OK;
}

}  // extern "C"
