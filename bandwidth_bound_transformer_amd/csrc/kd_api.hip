// kd_api.hip -- host side of the C ABI declared in include/kd.h.
//
// kd_init fixes everything ahead of the first step: the weight layout, the
// work plan, and every device buffer ("Why is real-time AI inference 56x more
// expensive?", section "decide everything ahead of time"). kd_step is then a
// single kernel launch on the caller's stream, with no allocation and no
// synchronisation ("keep the work resident on the GPU": per step the host
// only hands over the input and takes the output).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "kd.h"
#include "kd_batch_host.h"
#include "kd_device.h"
#include "kd_pack.h"

namespace {

constexpr int kRing = 13;
constexpr uint32_t kDefaultSpinUs = 2000000;  // 2 s
constexpr int kFlagStatus = 0, kFlagAbort = 1, kFlagSkip = 2, kFlagCancel = 3;

// Zero n 64-bit words (a kernel rather than a memset, so that a captured graph replays it reliably).
__global__ void clear_words_kernel(uint64_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

// ---- static scratch of kd_step_noalloc ----------------------------------------------------------
// 16 MiB per GPU, held until the process ends: word 0 is the abort word, the exchange words start
// at word kScratchHead. Host code never uses the array's name as an address: kd_init resolves the
// array's device address once per device and keeps it in g_scratch[device].
constexpr int64_t kScratchWords = (int64_t)2 << 20;
constexpr int64_t kScratchHead = 32;
__device__ __align__(256) uint64_t scratch[kScratchWords];

constexpr int kMaxDevices = 64;
struct StaticScratch {
  uint64_t* ptr = nullptr;  // device address of `scratch` on this device
  uint32_t next_tag = 0;    // tag base of the next call on this device (shared by every handle)
};
std::mutex g_scratch_mu;
StaticScratch g_scratch[kMaxDevices];

// With dev current: resolve the array's address once for this device. Returns false on failure.
bool resolve_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev].ptr) return true;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return false;
  g_scratch[dev].ptr = (uint64_t*)ptr;
  g_scratch[dev].next_tag = 0;
  return true;
}

// ---- plain stream read, the measured ceiling the decode kernels are compared with ---------------
// Workgroup b reads its own contiguous run of `per` 16-byte pieces, eight 4 KB rows of the run per
// iteration (each row one coalesced 16-byte load per thread), with non-temporal loads; the pieces
// past the last full run are swept grid-wide. The pieces are folded together and the fold is handed
// to an empty asm statement, so the compiler must keep every load. (On MI355X this shape read
// 7.1 TB/s over 4 GiB, against 6.2-7.0 TB/s for a grid-stride sweep.)
constexpr int kStreamU = 8;
constexpr int kStreamGrid = 8192;
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, int64_t per, int64_t n) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* q = (const u32x4*)p + (int64_t)blockIdx.x * per + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t it = 0; it < per; it += kStreamU * 256) {
    u32x4 v[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) v[u] = __builtin_nontemporal_load(q + it + u * 256);
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) acc ^= v[u];
  }
  const u32x4* r = (const u32x4*)p;
  for (int64_t i = (int64_t)gridDim.x * per + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    acc ^= __builtin_nontemporal_load(r + i);
  asm volatile("" ::"v"(acc.x ^ acc.y ^ acc.z ^ acc.w));
}

struct Buffers {
  uint8_t* blob = nullptr;
  uint8_t* embed = nullptr;
  uint8_t* norms = nullptr;
  float2* rope = nullptr;     // [S][hd/2] (cos, sin)
  float* scales = nullptr;    // fp8 or int8 weights: row scales (Dims::sc_*)
  uint64_t* ll = nullptr;
  uint32_t* flags = nullptr;  // [0] sticky status bits, [1] abort word, [2] tick skip flag (B > 1), [3] cancel word
};

void free_buffers(Buffers& b) {
  if (b.blob) (void)hipFree(b.blob);
  if (b.embed) (void)hipFree(b.embed);
  if (b.norms) (void)hipFree(b.norms);
  if (b.rope) (void)hipFree(b.rope);
  if (b.scales) (void)hipFree(b.scales);
  if (b.ll) (void)hipFree(b.ll);
  if (b.flags) (void)hipFree(b.flags);
  b = Buffers{};
}

typedef void (*KernelFn)(kd::Params);

// The one-step kernel, or (multi) the kernel that may run several steps per launch. int8: the
// one-byte matrix codes are int8 rather than E4M3.
KernelFn pick_kernel(int wbytes, int hd, bool multi, bool int8) {
  if (wbytes == 1 && hd == 128 && int8)
    return multi ? kd::decode_step_kernel<kRing, 1, 2, 128, true, true> : kd::decode_step_kernel<kRing, 1, 2, 128, false, true>;
  if (wbytes == 1 && hd == 128) return multi ? kd::decode_step_kernel<kRing, 1, 2, 128, true> : kd::decode_step_kernel<kRing, 1, 2, 128, false>;
  if (wbytes == 2 && hd == 128) return multi ? kd::decode_step_kernel<kRing, 2, 2, 128, true> : kd::decode_step_kernel<kRing, 2, 2, 128, false>;
  if (wbytes == 2 && hd == 64) return multi ? kd::decode_step_kernel<kRing, 2, 2, 64, true> : kd::decode_step_kernel<kRing, 2, 2, 64, false>;
  if (wbytes == 4 && hd == 128) return multi ? kd::decode_step_kernel<kRing, 4, 4, 128, true> : kd::decode_step_kernel<kRing, 4, 4, 128, false>;
  if (wbytes == 4 && hd == 64) return multi ? kd::decode_step_kernel<kRing, 4, 4, 64, true> : kd::decode_step_kernel<kRing, 4, 4, 64, false>;
  return nullptr;
}

}  // namespace

struct kd_handle {
  int device = 0;
  kd_config cfg{};
  kd::Dims m{};
  kd::LLLayout lo{};
  Buffers buf;
  KernelFn kernel = nullptr;        // one step per launch
  KernelFn kernel_multi = nullptr;  // several steps per launch (kd_generate)
  uint32_t next_tag = 0;  // tag base of the next launch (advances by steps * tag_stride)
  uint32_t spin_us = kDefaultSpinUs;
  int64_t lds_bytes = 0;
  uint64_t* trace = nullptr;
  hipStream_t ctl = nullptr;  // private non-blocking stream for cancel-word writes
  bool batched = false;  // B > 1: the lockstep-sessions path (kd_batch.h)
  kd::bt::BatchState bs;
  bool prefill = false;  // batch 1 with kd_prefill: the lockstep kernels, rows = prompt positions
  kd::bt::BatchState ps;
};

namespace {

bool dtype_ok(int32_t t) { return t == KD_DTYPE_F32 || t == KD_DTYPE_BF16; }
// one-byte matrix codes with a float32 scale per row
bool quantised(int32_t t) { return t == KD_DTYPE_FP8_E4M3 || t == KD_DTYPE_INT8; }
bool weight_dtype_ok(int32_t t) { return dtype_ok(t) || quantised(t); }
int dtype_bytes(int32_t t) { return quantised(t) ? 1 : (t == KD_DTYPE_BF16 ? 2 : 4); }

// Structural checks that need no device.
int check_config(const kd_config* c) {
  if (!c) return KD_ERR_INVALID_ARG;
  if (c->n_layers <= 0 || c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->ffn_dim <= 0 || c->vocab <= 0 || c->max_seq <= 0 || c->batch <= 0)
    return KD_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads != 0 || c->head_dim % 2 != 0) return KD_ERR_INVALID_ARG;
  if (!weight_dtype_ok(c->weight_dtype) || !dtype_ok(c->kv_dtype)) return KD_ERR_INVALID_ARG;
  if (!(c->norm_eps >= 0.f) || !(c->rope_base > 0.f)) return KD_ERR_INVALID_ARG;
  if (c->max_seq > (1 << 24) || c->vocab > (1 << 30)) return KD_ERR_INVALID_ARG;
  if (c->prefill_chunk < 0 || c->prefill_chunk > kd::bt::kMPrefill || c->prefill_chunk == 1) return KD_ERR_INVALID_ARG;
  return KD_OK;
}

// Limits of this implementation for a valid configuration, given the grid size.
int check_supported(const kd_config* c, const kd::Dims& m) {
  if (c->batch != 1) return KD_ERR_UNSUPPORTED;
  if (c->prefill_chunk > 0) {  // the lockstep kernels must take the shape
    kd_config pc = *c;
    pc.batch = c->prefill_chunk;
    const int rc = kd::bt::batch_check(&pc, kd::bt::kMPrefill);
    if (rc != KD_OK) return rc;
  }
  if (c->head_dim != 64 && c->head_dim != 128) return KD_ERR_UNSUPPORTED;
  // fp8 and int8 matrices come with bf16 embedding, gains and cache, and head_dim 128
  if (quantised(c->weight_dtype) ? (c->kv_dtype != KD_DTYPE_BF16 || c->head_dim != 128)
                                            : c->weight_dtype != c->kv_dtype)
    return KD_ERR_UNSUPPORTED;
  if (m.G > kd::kMaxGroup || (int64_t)m.G * m.hd > kd::kThreads) return KD_ERR_UNSUPPORTED;
  if (m.d > kd::kMaxDim || m.qdim > kd::kMaxDim || m.d % kd::down_block_rows(m) != 0) return KD_ERR_UNSUPPORTED;
  if ((int64_t)m.d * m.wbytes % kd::kPacketBytes || (int64_t)m.qdim * m.wbytes % kd::kPacketBytes) return KD_ERR_UNSUPPORTED;
  if (m.F % kd::ffn_unit(m) != 0 || m.F / kd::ffn_unit(m) < m.nwg) return KD_ERR_UNSUPPORTED;  // every workgroup owns an FFN slice
  // per-workgroup shares must fit the LDS arrays and the thread count
  const int64_t nrd_max = 2 * kd::ceil_div(m.d / 2, m.nwg);
  const int64_t nq_max = kd::ceil_div(m.nqkv, m.nwg);
  const int64_t nf_max = kd::ffn_unit(m) * kd::ceil_div(m.F / kd::ffn_unit(m), m.nwg);
  if (nrd_max > kd::kMaxRowsD || nq_max > kd::kThreads || nf_max > kd::kMaxSlice) return KD_ERR_UNSUPPORTED;
  if ((int64_t)m.nwg * nrd_max > kd::kStageWords || 2 * (int64_t)m.nwg > kd::kStageWords) return KD_ERR_UNSUPPORTED;
  // rows one wave's packet range can span, for every row-split tile of every workgroup
  auto max_rows = [&](auto rows_of, int64_t C) {
    int64_t worst = 0;
    for (int64_t w = 0; w < m.nwg; ++w) {
      const int64_t T = rows_of(w) * C;
      for (int v = 0; v < kd::kWaves; ++v) {
        const int64_t lo = kd::wave_lo(T, v), hi = kd::wave_lo(T, v + 1);
        if (hi > lo) worst = std::max(worst, (hi - 1) / C - lo / C + 1);
      }
    }
    return worst;
  };
  auto rows_qkv = [&](int64_t w) { return kd::part_lo(m.nqkv, m.nwg, w + 1) - kd::part_lo(m.nqkv, m.nwg, w); };
  auto rows_o = [&](int64_t w) { return 2 * (kd::part_lo(m.d / 2, m.nwg, w + 1) - kd::part_lo(m.d / 2, m.nwg, w)); };
  auto rows_gu = [&](int64_t w) { return 2 * (kd::ffn_lo(m, w + 1) - kd::ffn_lo(m, w)); };
  auto rows_lm = [&](int64_t w) { return kd::part_lo(m.V, m.nwg, w + 1) - kd::part_lo(m.V, m.nwg, w); };
  if (max_rows(rows_qkv, m.cd) > kd::kRowPart || max_rows(rows_o, m.cq) > kd::kRowPart ||
      max_rows(rows_gu, m.cd) > kd::kRowPart || max_rows(rows_lm, m.cd) > kd::kRowPart)
    return KD_ERR_UNSUPPORTED;
  // attention split at every position the cache can hold
  for (int32_t p = 0; p < c->max_seq; ++p) {
    const kd::AttPlan a = kd::att_plan(m, p);
    if (a.NC > kd::max_chunks(m)) return KD_ERR_UNSUPPORTED;
    if (kd::ceil_div(a.units, m.nwg) > kd::kMaxUnits) return KD_ERR_UNSUPPORTED;
    if ((int64_t)a.NC * (a.MS + 2) > kd::kStageWords || a.MS % 2 != 0) return KD_ERR_UNSUPPORTED;
    const int64_t pk = kd::ceil_div(a.CH, m.ppp);  // packets of one chunk
    if (kd::ceil_div(pk, kd::kWaves) * m.ppp > kd::kScorePos) return KD_ERR_UNSUPPORTED;
  }
  return KD_OK;
}

#define KD_TRY(expr)                                \
  do {                                              \
    if ((expr) != hipSuccess) { rc = KD_ERR_HIP; goto fail; } \
  } while (0)

}  // namespace

extern "C" {

const char* kd_strerror(int code) {
  switch (code) {
    case KD_OK: return "success";
    case KD_ERR_INVALID_ARG: return "invalid argument";
    case KD_ERR_UNSUPPORTED: return "configuration not supported by this library";
    case KD_ERR_NO_DEVICE: return "no HIP device available";
    case KD_ERR_OOM: return "device memory allocation failed";
    case KD_ERR_HIP: return "HIP runtime call failed";
    case KD_ERR_LAUNCH: return "kernel launch rejected";
    case KD_ERR_SCRATCH: return "the model needs more exchange memory than the static scratch of kd_step_noalloc holds (16 MiB)";
    default: return "unknown error code";
  }
}

int kd_kv_layout(const kd_config* cfg, size_t* bytes, size_t strides[6]) {
  const int rc0 = check_config(cfg);
  if (rc0 != KD_OK) return rc0;
  if (!bytes || !strides) return KD_ERR_INVALID_ARG;
  const size_t S = (size_t)kd::ceil_div((int64_t)cfg->max_seq + 7, 16) * 16;
  const size_t hd = (size_t)cfg->head_dim;
  strides[5] = 1;
  strides[4] = hd;
  strides[3] = S * hd;
  strides[2] = (size_t)cfg->n_kv_heads * strides[3];
  strides[1] = (size_t)cfg->batch * strides[2];
  strides[0] = 2 * strides[1];
  *bytes = (size_t)cfg->n_layers * strides[0] * (size_t)dtype_bytes(cfg->kv_dtype);
  return KD_OK;
}

int kd_init(const kd_config* cfg, const kd_weights* w, kd_handle** out) {
  if (!out) return KD_ERR_INVALID_ARG;
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc != KD_OK) return rc;
  if (!w || !w->embed || !w->layers || !w->final_norm || !w->lm_head) return KD_ERR_INVALID_ARG;
  const bool q8 = quantised(cfg->weight_dtype);  // one-byte codes with row scales (fp8 or int8)
  if (q8 && !w->s_lm_head) return KD_ERR_INVALID_ARG;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const kd_layer_weights& lw = w->layers[l];
    if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.ffn_norm || !lw.w_gate || !lw.w_up || !lw.w_down)
      return KD_ERR_INVALID_ARG;
    if (q8 && (!lw.s_wq || !lw.s_wk || !lw.s_wv || !lw.s_wo || !lw.s_gate || !lw.s_up || !lw.s_down))
      return KD_ERR_INVALID_ARG;
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return KD_ERR_NO_DEVICE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KD_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KD_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return KD_ERR_UNSUPPORTED;

  const int wb = dtype_bytes(cfg->weight_dtype), kb = dtype_bytes(cfg->kv_dtype);
  const int eb = q8 ? 2 : wb;  // embedding and norm gains
  const int nwg = prop.multiProcessorCount;
  if (cfg->batch > 1) {
    if (cfg->prefill_chunk != 0) return KD_ERR_INVALID_ARG;  // lockstep handles take no prefill
    rc = kd::bt::batch_check(cfg);
    if (rc != KD_OK) return rc;
    kd_handle* hb = new (std::nothrow) kd_handle();
    if (!hb) return KD_ERR_OOM;
    hb->device = dev;
    hb->cfg = *cfg;
    hb->batched = true;
    if (hipMalloc(&hb->buf.flags, 256) != hipSuccess) {
      delete hb;
      return KD_ERR_OOM;
    }
    if (hipMemset(hb->buf.flags, 0, 256) != hipSuccess) rc = KD_ERR_HIP;
    if (rc == KD_OK && hipStreamCreateWithFlags(&hb->ctl, hipStreamNonBlocking) != hipSuccess) rc = KD_ERR_HIP;
    if (rc == KD_OK) rc = kd::bt::batch_init(cfg, w, nwg, true, hb->bs);
    if (rc != KD_OK) {
      if (hb->ctl) (void)hipStreamDestroy(hb->ctl);
      free_buffers(hb->buf);
      delete hb;
      return rc;
    }
    *out = hb;
    return KD_OK;
  }
  const kd::Dims m = kd::make_dims(cfg->n_layers, cfg->d_model, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, cfg->ffn_dim,
                                   cfg->vocab, cfg->max_seq, nwg, wb, kb);
  rc = check_supported(cfg, m);
  if (rc != KD_OK) return rc;
  const bool int8 = cfg->weight_dtype == KD_DTYPE_INT8;
  KernelFn kern = pick_kernel(wb, cfg->head_dim, false, int8), kern_multi = pick_kernel(wb, cfg->head_dim, true, int8);
  if (!kern || !kern_multi) return KD_ERR_UNSUPPORTED;
  for (KernelFn k : {kern, kern_multi}) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)k, kd::kThreads, 0) != hipSuccess) return KD_ERR_HIP;
    if (occ < 1) return KD_ERR_UNSUPPORTED;
  }
  hipFuncAttributes fattr;
  if (hipFuncGetAttributes(&fattr, (const void*)kern) != hipSuccess) return KD_ERR_HIP;

  kd_handle* h = new (std::nothrow) kd_handle();
  if (!h) return KD_ERR_OOM;
  h->device = dev;
  h->cfg = *cfg;
  h->m = m;
  h->lo = kd::ll_layout(m);
  h->kernel = kern;
  h->kernel_multi = kern_multi;
  h->lds_bytes = (int64_t)fattr.sharedSizeBytes;
  h->next_tag = kd::tag_stride(m);

  uint8_t* tmp = nullptr;
  {
    const int64_t d = m.d;
    const size_t blob_bytes = (size_t)m.blob_elems * wb;
    if (hipMalloc(&h->buf.blob, blob_bytes) != hipSuccess) { rc = KD_ERR_OOM; goto fail; }
    if (hipMalloc(&h->buf.embed, (size_t)m.V * d * eb) != hipSuccess) { rc = KD_ERR_OOM; goto fail; }
    if (hipMalloc(&h->buf.norms, (size_t)(2 * m.L + 1) * d * eb) != hipSuccess) { rc = KD_ERR_OOM; goto fail; }
    if (q8 && hipMalloc(&h->buf.scales, (size_t)kd::scale_layout(m).total * sizeof(float)) != hipSuccess) { rc = KD_ERR_OOM; goto fail; }
    if (hipMalloc(&h->buf.ll, (size_t)h->lo.total * 8) != hipSuccess) { rc = KD_ERR_OOM; goto fail; }
    if (hipMalloc(&h->buf.rope, (size_t)m.S * (m.hd / 2) * sizeof(float2)) != hipSuccess) { rc = KD_ERR_OOM; goto fail; }
    if (hipMalloc(&h->buf.flags, 256) != hipSuccess) { rc = KD_ERR_OOM; goto fail; }
    if (hipMalloc(&tmp, (size_t)2 * m.F * d * wb) != hipSuccess) { rc = KD_ERR_OOM; goto fail; }
    KD_TRY(hipMemset(h->buf.ll, 0, (size_t)h->lo.total * 8));
    KD_TRY(hipMemset(h->buf.flags, 0, 256));
    KD_TRY(hipStreamCreateWithFlags(&h->ctl, hipStreamNonBlocking));
    // kd_step_noalloc's scratch on this device (if this fails, that entry point reports KD_ERR_HIP)
    (void)resolve_scratch(dev);
    const size_t row = (size_t)d * wb, erow = (size_t)d * eb;
    const kd::ScaleLayout sl = kd::scale_layout(m);
    std::vector<float> sc(q8 ? (size_t)sl.total : 0);
    for (int l = 0; l < m.L; ++l) {
      const kd_layer_weights& lw = w->layers[l];
      uint8_t* lay = h->buf.blob + (size_t)l * m.layer_elems * wb;
      KD_TRY(hipMemcpy(lay + m.off_qkv * wb, lw.wq, (size_t)m.qdim * row, hipMemcpyHostToDevice));
      KD_TRY(hipMemcpy(lay + (m.off_qkv + (int64_t)m.qdim * d) * wb, lw.wk, (size_t)m.kvdim * row, hipMemcpyHostToDevice));
      KD_TRY(hipMemcpy(lay + (m.off_qkv + (int64_t)(m.qdim + m.kvdim) * d) * wb, lw.wv, (size_t)m.kvdim * row, hipMemcpyHostToDevice));
      KD_TRY(hipMemcpy(lay + m.off_o * wb, lw.wo, (size_t)d * m.qdim * wb, hipMemcpyHostToDevice));
      KD_TRY(hipMemcpy(tmp, lw.w_gate, (size_t)m.F * row, hipMemcpyHostToDevice));
      KD_TRY(hipMemcpy(tmp + (size_t)m.F * row, lw.w_up, (size_t)m.F * row, hipMemcpyHostToDevice));
      if (wb == 1)
        hipLaunchKernelGGL(kd::pack_gate_up_kernel<uint8_t>, dim3(4096), dim3(256), 0, 0, (uint8_t*)(lay + m.off_gu * wb),
                           (const uint8_t*)tmp, (const uint8_t*)(tmp + (size_t)m.F * row), m);
      else if (wb == 2)
        hipLaunchKernelGGL(kd::pack_gate_up_kernel<uint16_t>, dim3(4096), dim3(256), 0, 0, (uint16_t*)(lay + m.off_gu * wb),
                           (const uint16_t*)tmp, (const uint16_t*)(tmp + (size_t)m.F * row), m);
      else
        hipLaunchKernelGGL(kd::pack_gate_up_kernel<float>, dim3(4096), dim3(256), 0, 0, (float*)(lay + m.off_gu * wb),
                           (const float*)tmp, (const float*)(tmp + (size_t)m.F * row), m);
      KD_TRY(hipGetLastError());
      KD_TRY(hipDeviceSynchronize());
      KD_TRY(hipMemcpy(tmp, lw.w_down, (size_t)d * m.F * wb, hipMemcpyHostToDevice));
      if (wb == 1)
        hipLaunchKernelGGL(kd::pack_down_kernel<uint8_t>, dim3(4096), dim3(256), 0, 0, (uint8_t*)(lay + m.off_d * wb),
                           (const uint8_t*)tmp, m);
      else if (wb == 2)
        hipLaunchKernelGGL(kd::pack_down_kernel<uint16_t>, dim3(4096), dim3(256), 0, 0, (uint16_t*)(lay + m.off_d * wb),
                           (const uint16_t*)tmp, m);
      else
        hipLaunchKernelGGL(kd::pack_down_kernel<float>, dim3(4096), dim3(256), 0, 0, (float*)(lay + m.off_d * wb),
                           (const float*)tmp, m);
      KD_TRY(hipGetLastError());
      KD_TRY(hipDeviceSynchronize());
      KD_TRY(hipMemcpy(h->buf.norms + (size_t)(2 * l) * erow, lw.attn_norm, erow, hipMemcpyHostToDevice));
      KD_TRY(hipMemcpy(h->buf.norms + (size_t)(2 * l + 1) * erow, lw.ffn_norm, erow, hipMemcpyHostToDevice));
      if (q8) {
        // row scales in the rows' packed order: QKV (q, k, v), O, each workgroup's [gate; up] slice, down
        float* L0 = sc.data() + (size_t)l * sl.layer;
        std::memcpy(L0, lw.s_wq, sizeof(float) * m.qdim);
        std::memcpy(L0 + m.qdim, lw.s_wk, sizeof(float) * m.kvdim);
        std::memcpy(L0 + m.qdim + m.kvdim, lw.s_wv, sizeof(float) * m.kvdim);
        std::memcpy(L0 + sl.o, lw.s_wo, sizeof(float) * d);
        for (int64_t wg = 0; wg < m.nwg; ++wg) {
          const int64_t f0 = kd::ffn_lo(m, wg), nf = kd::ffn_lo(m, wg + 1) - f0;
          std::memcpy(L0 + sl.gu + 2 * f0, lw.s_gate + f0, sizeof(float) * nf);
          std::memcpy(L0 + sl.gu + 2 * f0 + nf, lw.s_up + f0, sizeof(float) * nf);
        }
        std::memcpy(L0 + sl.d, lw.s_down, sizeof(float) * d);
      }
    }
    KD_TRY(hipMemcpy(h->buf.norms + (size_t)(2 * m.L) * erow, w->final_norm, erow, hipMemcpyHostToDevice));
    KD_TRY(hipMemcpy(h->buf.blob + (size_t)m.off_lm * wb, w->lm_head, (size_t)m.V * row, hipMemcpyHostToDevice));
    KD_TRY(hipMemcpy(h->buf.embed, w->embed, (size_t)m.V * erow, hipMemcpyHostToDevice));
    if (q8) {
      std::memcpy(sc.data() + sl.lm, w->s_lm_head, sizeof(float) * m.V);
      KD_TRY(hipMemcpy(h->buf.scales, sc.data(), sc.size() * sizeof(float), hipMemcpyHostToDevice));
    }
    {
      // RoPE: pair (i, i + hd/2) turns by position * base^(-2i/hd); angles, cos and sin in float64
      const int half = m.hd / 2;
      std::vector<float2> tab((size_t)m.S * half);
      std::vector<double> theta(half);
      for (int i = 0; i < half; ++i) theta[i] = std::pow((double)cfg->rope_base, -2.0 * (double)i / (double)m.hd);
      for (int64_t pos = 0; pos < m.S; ++pos)
        for (int i = 0; i < half; ++i) {
          const double ang = (double)pos * theta[i];
          tab[(size_t)pos * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
        }
      KD_TRY(hipMemcpy(h->buf.rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice));
    }
    KD_TRY(hipDeviceSynchronize());
    (void)hipFree(tmp);
    tmp = nullptr;
  }
  if (cfg->prefill_chunk > 0) {
    // the prefill engine: the lockstep kernels with prefill_chunk rows (weights in their tile layout)
    kd_config pc = *cfg;
    pc.batch = cfg->prefill_chunk;
    rc = kd::bt::batch_init(&pc, w, nwg, false, h->ps);
    if (rc != KD_OK) goto fail;
    h->prefill = true;
  }
  *out = h;
  return KD_OK;

fail:
  if (tmp) (void)hipFree(tmp);
  if (h->ctl) (void)hipStreamDestroy(h->ctl);
  free_buffers(h->buf);
  if (h->prefill) kd::bt::batch_free(h->ps);
  delete h;
  return rc;
}

}  // extern "C"

namespace {

// Tag bases for a launch of n steps from the counter *next (advanced past them). A range never
// wraps past zero: when it would, the counter restarts and *clear is set, and the caller clears
// the exchange words first, so no word left from before can carry a tag of the new range.
uint32_t take_tags(uint32_t* next, uint32_t stride, int n, bool* clear) {
  const uint64_t need = (uint64_t)stride * (uint64_t)n;
  *clear = false;
  if ((uint64_t)*next + need >= (1ull << 32)) {
    *next = stride;
    *clear = true;
  }
  const uint32_t t = *next;
  *next = (uint32_t)(t + need);
  return t;
}

// Launch n steps of the batch-1 kernel with the exchange words at ll, the abort word at abortf and
// tags from tag0 on.
int launch_steps_at(kd_handle* h, uint64_t* ll, uint32_t* abortf, uint32_t tag0, int n, int32_t* tokens,
                    int32_t* positions, void* kv, float* logits, int32_t* out_tokens, uint32_t* progress,
                    hipStream_t stream) {
  kd::Params P{};
  P.blob = h->buf.blob;
  P.embed = h->buf.embed;
  P.norms = h->buf.norms;
  P.scales = h->buf.scales;
  P.rope = h->buf.rope;
  P.ll = ll;
  P.lo = h->lo;
  P.kv = (uint8_t*)kv;
  P.tokens = tokens;
  P.positions = positions;
  P.logits = logits;
  P.flags = h->buf.flags;
  P.abortf = abortf;
  P.trace = h->trace;
  P.out_tokens = out_tokens;
  P.progress = progress;
  P.spin_us = h->spin_us;
  P.tag0 = tag0;
  P.n_steps = n;
  P.max_seq = h->cfg.max_seq;
  P.eps = h->cfg.norm_eps;
  P.m = h->m;
  void* args[] = {&P};
  // One workgroup per compute unit, and a workgroup needs most of a CU's LDS, so on an idle
  // device the whole grid is resident at once. If another kernel holds CUs, the waits between
  // workgroups time out and the launch ends with KD_STATUS_SYNC_TIMEOUT instead of hanging.
  const hipError_t e =
      hipLaunchKernel((const void*)(n > 1 ? h->kernel_multi : h->kernel), dim3(h->m.nwg), dim3(kd::kThreads), args, 0, stream);
  return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

// The same with the handle's own exchange words and tag counter.
int launch_steps(kd_handle* h, int n, int32_t* tokens, int32_t* positions, void* kv, float* logits, int32_t* out_tokens,
                 uint32_t* progress, hipStream_t stream) {
  bool clear = false;
  const uint32_t tag0 = take_tags(&h->next_tag, kd::tag_stride(h->m), n, &clear);
  if (clear) {
    hipLaunchKernelGGL(clear_words_kernel, dim3(256), dim3(256), 0, stream, h->buf.ll, (int64_t)h->lo.total);
    if (hipGetLastError() != hipSuccess) return KD_ERR_LAUNCH;
  }
  return launch_steps_at(h, h->buf.ll, h->buf.flags + kFlagAbort, tag0, n, tokens, positions, kv, logits, out_tokens,
                         progress, stream);
}

// Makes h's device current for the lifetime of the guard, then restores the caller's.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = prev == dev || hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

}  // namespace

extern "C" {

int kd_step(kd_handle* h, int32_t* tokens, int32_t* positions, void* kv, float* logits, void* stream) {
  if (!h || !tokens || !positions || !kv) return KD_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  if (!g.ok) return KD_ERR_HIP;
  if (h->batched)
    return kd::bt::batch_step(h->bs, tokens, positions, kv, logits, (hipStream_t)stream, h->buf.flags, nullptr, nullptr, 0);
  return launch_steps(h, 1, tokens, positions, kv, logits, nullptr, nullptr, (hipStream_t)stream);
}

int kd_step_noalloc(kd_handle* h, int32_t* tokens, int32_t* positions, void* kv, float* logits, void* stream) {
  if (!h || !tokens || !positions || !kv) return KD_ERR_INVALID_ARG;
  if (h->batched) return KD_ERR_UNSUPPORTED;
  if (h->device < 0 || h->device >= kMaxDevices) return KD_ERR_HIP;
  if (h->lo.total > kScratchWords - kScratchHead) return KD_ERR_SCRATCH;
  DeviceGuard g(h->device);
  if (!g.ok) return KD_ERR_HIP;
  uint64_t* base = nullptr;
  uint32_t tag0 = 0;
  bool clear = false;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    base = g_scratch[h->device].ptr;
    if (!base) return KD_ERR_HIP;
    uint32_t& next = g_scratch[h->device].next_tag;
    if (next == 0) next = kd::tag_stride(h->m);
    tag0 = take_tags(&next, kd::tag_stride(h->m), 1, &clear);
  }
  if (clear) {  // the device's tags start over: no word of the array may keep an old tag
    hipLaunchKernelGGL(clear_words_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream, base, kScratchWords);
    if (hipGetLastError() != hipSuccess) return KD_ERR_LAUNCH;
  }
  return launch_steps_at(h, base + kScratchHead, (uint32_t*)base, tag0, 1, tokens, positions, kv, logits, nullptr, nullptr,
                         (hipStream_t)stream);
}

int kd_prefill(kd_handle* h, const int32_t* prompt, int32_t n, int32_t* tokens, int32_t* positions, void* kv,
               float* logits, void* stream) {
  if (!h || !prompt || !tokens || !positions || !kv || n < 1) return KD_ERR_INVALID_ARG;
  if (!h->prefill) return KD_ERR_UNSUPPORTED;
  DeviceGuard g(h->device);
  if (!g.ok) return KD_ERR_HIP;
  return kd::bt::batch_prefill(h->ps, prompt, n, tokens, positions, kv, logits, (hipStream_t)stream, h->buf.flags);
}

int kd_generate(kd_handle* h, int32_t n_steps, int32_t* tokens, int32_t* positions, void* kv, int32_t* out_tokens,
                float* logits, uint32_t* progress, void* stream) {
  if (!h || !tokens || !positions || !kv || n_steps < 1) return KD_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  if (!g.ok) return KD_ERR_HIP;
  if (h->batched) {
    // B > 1: the ticks' kernel sequences back to back on the stream, tokens fed back on the device
    const size_t per = (size_t)h->bs.B * h->bs.V;
    for (int s = 0; s < n_steps; ++s) {
      const int rc = kd::bt::batch_step(h->bs, tokens, positions, kv, logits ? logits + s * per : nullptr,
                                        (hipStream_t)stream, h->buf.flags, out_tokens ? out_tokens + (size_t)s * h->bs.B : nullptr,
                                        progress, (uint32_t)(s + 1));
      if (rc != KD_OK) return rc;
    }
    return KD_OK;
  }
  return launch_steps(h, n_steps, tokens, positions, kv, logits, out_tokens, progress, (hipStream_t)stream);
}

int kd_control(kd_handle* h, int32_t op, int64_t value) {
  if (!h) return KD_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  if (!g.ok) return KD_ERR_HIP;
  switch (op) {
    case KD_CTRL_CANCEL: {
      // written on the handle's own non-blocking stream, so it lands while a launch runs
      static const uint32_t kOne = 1, kZero = 0;
      if (hipMemcpyAsync(h->buf.flags + kFlagCancel, value ? &kOne : &kZero, 4, hipMemcpyHostToDevice, h->ctl) != hipSuccess)
        return KD_ERR_HIP;
      return hipStreamSynchronize(h->ctl) == hipSuccess ? KD_OK : KD_ERR_HIP;
    }
    case KD_CTRL_WAIT_LIMIT_US:
      if (value < 0 || value > 60000000) return KD_ERR_INVALID_ARG;
      h->spin_us = (uint32_t)value;
      return KD_OK;
    default:
      return KD_ERR_INVALID_ARG;
  }
}

int kd_device_status(kd_handle* h, uint32_t* bits, int clear) {
  if (!h || !bits) return KD_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  if (!g.ok) return KD_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return KD_ERR_HIP;
  uint32_t f = 0;
  if (hipMemcpy(&f, h->buf.flags + kFlagStatus, sizeof(f), hipMemcpyDeviceToHost) != hipSuccess) return KD_ERR_HIP;
  *bits = f;
  if (clear && hipMemset(h->buf.flags + kFlagStatus, 0, sizeof(f)) != hipSuccess) return KD_ERR_HIP;
  return KD_OK;
}

void kd_destroy(kd_handle* h) {
  if (!h) return;
  {
    DeviceGuard g(h->device);
    (void)hipDeviceSynchronize();
    if (h->ctl) (void)hipStreamDestroy(h->ctl);
    free_buffers(h->buf);
    if (h->batched) kd::bt::batch_free(h->bs);
    if (h->prefill) kd::bt::batch_free(h->ps);
  }
  delete h;
}

int kd_stream_read(const void* buf, size_t bytes, void* stream) {
  if (!buf || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0) return KD_ERR_INVALID_ARG;
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t row = (int64_t)kStreamU * 256;
  const int64_t per = n / kStreamGrid / row * row;  // whole iterations per workgroup; the rest grid-wide
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamGrid), dim3(256), 0, (hipStream_t)stream, (const uint4*)buf, per, n);
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

int kd_trace(kd_handle* h, uint64_t* dev_buf, int64_t words, int64_t* stride) {
  if (!h) return KD_ERR_INVALID_ARG;
  if (h->batched || h->m.L > kd::kTraceMaxLayers) return KD_ERR_UNSUPPORTED;
  const int64_t st = kd::trace_stride(h->m.L);
  if (stride) *stride = st;
  if (!dev_buf) {
    h->trace = nullptr;
    return KD_OK;
  }
  if (words < st * h->m.nwg) return KD_ERR_INVALID_ARG;
  h->trace = dev_buf;
  return KD_OK;
}

int kd_get_info(kd_handle* h, int64_t info[8]) {
  if (!h || !info) return KD_ERR_INVALID_ARG;
  for (int i = 0; i < 8; ++i) info[i] = 0;
  if (h->batched) {
    const kd::bt::BatchState& b = h->bs;
    info[0] = 0;
    info[1] = kd::bt::gemm_threads(h->bs.MT);
    // packed weights (bf16 tiles, or one-byte tiles and their row scales), embedding, norm gains
    info[2] = (b.q ? (int64_t)(b.w_lm + (size_t)b.V * b.d) + ((int64_t)b.L * (int64_t)b.srows + b.V) * 4
                   : (int64_t)(b.w_lm + (size_t)b.V * b.d) * 2) +
              (int64_t)b.V * b.d * 2 + (int64_t)(2 * b.L + 1) * b.d * 2;
    info[5] = kd::bt::batch_kernels_per_tick(b);
    info[6] = b.g_qkv.KS | (b.g_o.KS << 8) | (b.g_gu.KS << 16) | (b.g_d.KS << 24);
    info[7] = b.CH;
    return KD_OK;
  }
  info[0] = h->m.nwg;
  info[1] = kd::kThreads;
  info[2] = h->m.blob_elems * h->m.wbytes + (int64_t)h->m.V * h->m.d * kd::embed_bytes(h->m) +
            (int64_t)(2 * h->m.L + 1) * h->m.d * kd::embed_bytes(h->m) + (h->buf.scales ? kd::scale_layout(h->m).total * 4 : 0);
  info[3] = h->lds_bytes;
  info[4] = kRing;
  info[5] = h->prefill ? h->ps.B : 0;
  return KD_OK;
}

}  // extern "C"
