// C ABI: argument checking on the host, then kernel dispatch.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tq_kernels.h"

namespace tq {

namespace {
thread_local std::string g_last_error;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int32_t kKnownLayerFlags = TQ_LAYER_BETA_CODEBOOK | TQ_LAYER_DITHER | TQ_LAYER_VALUE_QJL;
// The dithered variant is defined for the randomized Hadamard rotation and
// keys without QJL.
bool dither_ok(int32_t flags, int32_t rot, int32_t k_qjl) {
  return !(flags & TQ_LAYER_DITHER) ||
         (rot == TQ_ROT_HADAMARD && k_qjl == 0 && !(flags & TQ_LAYER_VALUE_QJL));
}

// Whether rows of tensor `which` carry QJL sign bits and residual norms.
bool rows_qjl(const tq_layer* L, int which) {
  return which == TQ_KEYS ? L->k_qjl != 0 : (L->flags & TQ_LAYER_VALUE_QJL) != 0;
}

// The kernels address one sequence of a cache array through 32-bit byte
// offsets (buffer descriptors, with a few hundred keys of read-ahead past the
// last block), so each array of a sequence must stay below 2^31 bytes with
// margin.  The code array is the largest (d * bits / 8 bytes per token, at
// least the d / 8 of the sign bits).
constexpr int64_t kSeqBytesMax = ((int64_t)1 << 31) - ((int64_t)1 << 20);
bool seq_bytes_ok(int d, int bits, int64_t cap) { return cap <= kSeqBytesMax / ((int64_t)d * bits / 8); }

struct Plan {  // split-K plan of one decode call
  bool mfma;     // matrix-core kernel (else the reference kernels)
  bool wide;     // the many-rows matrix-core kernel
  int nsplit;
  int waves;     // per workgroup (matrix-core kernel)
  int64_t keys_per_split;
  int64_t rows_total;
  size_t off_qrot, off_qproj, off_part, total;
};

// dither: the dithered variant, which the many-rows kernel does not implement;
// vqjl: values with QJL, which only the reference kernels implement (their
// partial rows also carry the sum of the values' QJL terms).
Plan decode_plan(int d, int qjl, int dither, int vqjl, int B, int Hq, int Hkv, int Tq, int64_t N) {
  Plan p{};
  const int64_t seqs = (int64_t)B * Hkv;
  p.mfma = !vqjl && mfma_decode_supports(d, Hq / Hkv * Tq);
  if (p.mfma) {
    // Work in blocks of 32 keys.  A workgroup serves up to 4 (or 8) query rows
    // of one KV head; split the keys so that the workgroups fill the chip's 256
    // CUs once (as many waves on each as the registers allow) -- a second round
    // of workgroups costs more in set-up and tail than it gains -- while giving
    // each wave at least 4 blocks.  The plan depends on the shape only, so the
    // workspace size does too.
    const int64_t blocks = (N + 31) / 32;
    if (!dither && decode_is_wide(d, Hq / Hkv * Tq)) {
      // 4-wave workgroups of 64 query rows (16 per wave), kWideGroupsPerCU
      // per CU; split the keys so that the workgroups fill the 256 CUs once,
      // each split at least 8 blocks.
      const int64_t groups = seqs * ((Hq / Hkv * Tq + kWideRowsPerGroup - 1) / kWideRowsPerGroup);
      int64_t want = (256 * kWideGroupsPerCU + groups - 1) / groups;
      const int64_t max_split = (blocks + 7) / 8;
      if (want > max_split) want = max_split;
      if (want > 1024) want = 1024;
      if (want < 1) want = 1;
      const int64_t bps = (blocks + want - 1) / want;
      p.wide = true;
      p.waves = 4;
      p.keys_per_split = bps * 32;
      p.nsplit = (int)((blocks + bps - 1) / bps);
    } else {
    const int rw = decode_rows_per_group(Hq / Hkv * Tq);
    const int64_t groups = seqs * ((Hq / Hkv * Tq + rw - 1) / rw);
    const int simd_waves = decode_simd_waves(d, qjl, rw);
    auto split_keys = [&](int waves) {
      const int64_t target = 256 * 4 * simd_waves / waves;
      int64_t want = (target + groups - 1) / groups;
      const int64_t max_split = (blocks + 4 * waves - 1) / (4 * waves);
      if (want > max_split) want = max_split;
      if (want > 1024) want = 1024;  // the combine kernel keeps one weight per split in LDS
      if (want < 1) want = 1;
      const int64_t bps = (blocks + want - 1) / want;
      p.waves = waves;
      p.keys_per_split = bps * 32;
      p.nsplit = (int)((blocks + bps - 1) / bps);
    };
    // Workgroups of 4 waves, two per CU where the registers allow.  When they
    // fill every CU but leave each wave fewer than 16 blocks, the set-up (code
    // tables and query rotation, once per workgroup) weighs on the short key
    // loop, and one 8-wave workgroup per CU, which does it once with twice the
    // threads, is faster (4-row groups only).
    split_keys(4);
    if (simd_waves == 2 && rw == 4 && groups <= 256 && groups * p.nsplit >= 512 && p.keys_per_split < 4 * 16 * 32)
      split_keys(8);
    }
  } else {
    int64_t want = (2048 + seqs - 1) / seqs;
    const int64_t max_split = (N + 63) / 64;
    if (want > max_split) want = max_split;
    if (want > 1024) want = 1024;
    if (want < 1) want = 1;
    p.keys_per_split = (N + want - 1) / want;
    p.nsplit = (int)((N + p.keys_per_split - 1) / p.keys_per_split);
  }
  p.rows_total = (int64_t)B * Hq * Tq;
  size_t o = 0;
  // The reference path rotates the query rows into the workspace first; the
  // matrix-core kernel does it on chip.
  const size_t qbytes = p.mfma ? 0 : (size_t)p.rows_total * d * sizeof(float);
  p.off_qrot = o;  o = align_up(o + qbytes, 256);
  p.off_qproj = o; o = align_up(o + qbytes, 256);
  p.off_part = o;  o = align_up(o + (size_t)p.nsplit * p.rows_total * ((vqjl ? 2 * d : d) + kPartPad) * sizeof(float), 256);
  p.total = o;
  return p;
}

tq_status check_layer(const tq_layer* L) {
  if (!L) return fail(TQ_ERR_INVALID_ARG, "layer is NULL");
  if (!supported_d(L->d)) return fail(TQ_ERR_UNSUPPORTED, "d must be 64, 128 or 256");
  if (L->rot != TQ_ROT_HAAR && L->rot != TQ_ROT_HADAMARD)
    return fail(TQ_ERR_INVALID_ARG, "rot must be TQ_ROT_HAAR or TQ_ROT_HADAMARD");
  if (L->k_bits < 1 || L->k_bits > 4 || L->v_bits < 1 || L->v_bits > 4)
    return fail(TQ_ERR_INVALID_ARG, "bit widths must be 1..4");
  if (L->k_qjl != 0 && L->k_qjl != 1) return fail(TQ_ERR_INVALID_ARG, "k_qjl must be 0 or 1");
  if (L->flags & ~kKnownLayerFlags) return fail(TQ_ERR_INVALID_ARG, "unknown layer flags");
  if (!dither_ok(L->flags, L->rot, L->k_qjl))
    return fail(TQ_ERR_INVALID_ARG, "TQ_LAYER_DITHER needs the Hadamard rotation and keys and values without QJL");
  if (!L->blob) return fail(TQ_ERR_INVALID_ARG, "layer blob is NULL");
  if (L->blob_bytes < blob_layout(L->d).total) return fail(TQ_ERR_INVALID_ARG, "layer blob too small");
  return TQ_OK;
}

tq_status check_cache(const tq_layer* L, int which, const tq_cache* c, const char* name) {
  const std::string n(name);
  if (!c) return fail(TQ_ERR_INVALID_ARG, n + " cache is NULL");
  if (c->seqs < 0) return fail(TQ_ERR_INVALID_ARG, n + ": seqs must be >= 0");
  if (c->cap <= 0 || c->cap % 8) return fail(TQ_ERR_INVALID_ARG, n + ": cap must be a positive multiple of 8");
  const bool qjl = rows_qjl(L, which);
  if (!c->idx || !c->norm) return fail(TQ_ERR_INVALID_ARG, n + ": idx and norm are required");
  if (qjl && (!c->sign || !c->rnorm))
    return fail(TQ_ERR_INVALID_ARG, n + ": rows with QJL need sign and rnorm");
  if (!aligned16(c->idx) || !aligned16(c->norm) || (qjl && (!aligned16(c->sign) || !aligned16(c->rnorm))))
    return fail(TQ_ERR_ALIGNMENT, n + ": cache pointers must be 16-byte aligned");
  if (!seq_bytes_ok(L->d, which == TQ_KEYS ? L->k_bits : L->v_bits, c->cap))
    return fail(TQ_ERR_UNSUPPORTED, n + ": cap * d * bits / 8 must stay below 2^31 - 2^20 bytes per sequence");
  return TQ_OK;
}

const float* blob_f(const tq_layer* L, size_t off) {
  return reinterpret_cast<const float*>(static_cast<const unsigned char*>(L->blob) + off);
}
const void* blob_p(const tq_layer* L, size_t off) {
  return static_cast<const unsigned char*>(L->blob) + off;
}

tq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TQ_OK;
  return fail(TQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Checks of tq_dequantize (prod: also the QJL fields of tq_dequantize_prod).
tq_status check_dequantize(const tq_layer* layer, int32_t which, const tq_cache* cache, int64_t n, const void* out,
                           int32_t out_dtype, bool prod) {
  tq_status s = check_layer(layer);
  if (s != TQ_OK) return s;
  if (which != TQ_KEYS && which != TQ_VALUES) return fail(TQ_ERR_INVALID_ARG, "which must be TQ_KEYS or TQ_VALUES");
  if (out_dtype != TQ_F32 && out_dtype != TQ_F16) return fail(TQ_ERR_INVALID_ARG, "out_dtype must be TQ_F32 or TQ_F16");
  if (!cache || !cache->idx || !cache->norm) return fail(TQ_ERR_INVALID_ARG, "cache idx and norm are required");
  if (cache->seqs < 0 || cache->cap <= 0 || cache->cap % 8)
    return fail(TQ_ERR_INVALID_ARG, "cache needs seqs >= 0 and cap a positive multiple of 8");
  if (!aligned16(cache->idx) || !aligned16(cache->norm)) return fail(TQ_ERR_ALIGNMENT, "cache pointers must be 16-byte aligned");
  if (prod) {
    if (!rows_qjl(layer, which))
      return fail(TQ_ERR_INVALID_ARG,
                  "the two-stage reconstruction needs rows with QJL (keys with k_qjl = 1, values with "
                  "TQ_LAYER_VALUE_QJL)");
    if (!cache->sign || !cache->rnorm) return fail(TQ_ERR_INVALID_ARG, "rows with QJL need sign and rnorm");
    if (!aligned16(cache->sign) || !aligned16(cache->rnorm))
      return fail(TQ_ERR_ALIGNMENT, "cache pointers must be 16-byte aligned");
  }
  if (n < 0 || n > cache->cap) return fail(TQ_ERR_INVALID_ARG, "n must be in [0, cap]");
  if (cache->seqs > 65535) return fail(TQ_ERR_UNSUPPORTED, "at most 65535 sequences per call");
  if (!seq_bytes_ok(layer->d, which == TQ_KEYS ? layer->k_bits : layer->v_bits, cache->cap))
    return fail(TQ_ERR_UNSUPPORTED, "cap * d * bits / 8 must stay below 2^31 - 2^20 bytes per sequence");
  if (n > 0 && cache->seqs > 0) {
    if (!out) return fail(TQ_ERR_INVALID_ARG, "out is NULL");
    if (!aligned16(out)) return fail(TQ_ERR_ALIGNMENT, "out must be 16-byte aligned");
  }
  return TQ_OK;
}

DequantArgs dequant_args(const tq_layer* layer, int32_t which, const tq_cache* cache, int64_t n, void* out,
                         int32_t out_dtype) {
  const BlobLayout BL = blob_layout(layer->d);
  DequantArgs a{};
  a.idx = cache->idx;
  a.norm = cache->norm;
  a.seqs = cache->seqs;
  a.n = n;
  a.cap = cache->cap;
  a.d = layer->d;
  a.bits = which == TQ_KEYS ? layer->k_bits : layer->v_bits;
  a.value_layout = which == TQ_VALUES;
  a.R = blob_f(layer, BL.rot);
  a.Rt = blob_f(layer, BL.rot_t);
  a.cent = blob_f(layer, BL.codebook) + (which == TQ_KEYS ? 0 : 2 * kMaxLevels);
  a.rot = layer->rot;
  a.dsign = blob_f(layer, BL.signs);
  a.out = out;
  a.out_dtype = out_dtype;
  a.dither = (layer->flags & TQ_LAYER_DITHER) != 0;
  a.dither_s0 = dither_stream_start(layer->seed, which == TQ_KEYS ? kDitherTagKeys : kDitherTagValues);
  a.dither_w = blob_f(layer, BL.scales) + (which == TQ_KEYS ? 4 : 5);
  a.cscale = blob_f(layer, BL.scales) + (which == TQ_KEYS ? 0 : 1);
  return a;
}

// Everything tq_attn_decode checks before it looks at the workspace; fills the
// split plan.  Host only.
tq_status check_decode(const tq_layer* layer, const void* q, int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                       int32_t Tq, int64_t N, int32_t causal, const tq_cache* K, const tq_cache* V,
                       const float* out, const float* scores, Plan* plan) {
  tq_status s = check_layer(layer);
  if (s != TQ_OK) return s;
  if (q_dtype != TQ_F32 && q_dtype != TQ_F16) return fail(TQ_ERR_INVALID_ARG, "q_dtype must be TQ_F32 or TQ_F16");
  if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1) return fail(TQ_ERR_INVALID_ARG, "B, Hq, Hkv and Tq must be >= 1");
  if (Hq % Hkv) return fail(TQ_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (N < 1) return fail(TQ_ERR_INVALID_ARG, "N must be >= 1");
  if (causal != 0 && causal != 1) return fail(TQ_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (causal && Tq > N) return fail(TQ_ERR_INVALID_ARG, "causal decode needs Tq <= N");
  if ((s = check_cache(layer, TQ_KEYS, K, "K")) != TQ_OK) return s;
  if ((s = check_cache(layer, TQ_VALUES, V, "V")) != TQ_OK) return s;
  if (K->seqs != (int64_t)B * Hkv || V->seqs != (int64_t)B * Hkv)
    return fail(TQ_ERR_INVALID_ARG, "K and V must hold B*Hkv sequences");
  if (K->cap != V->cap) return fail(TQ_ERR_INVALID_ARG, "K and V must have the same capacity");
  if (N > K->cap) return fail(TQ_ERR_INVALID_ARG, "N exceeds the cache capacity");
  if (!q || !out) return fail(TQ_ERR_INVALID_ARG, "q and out are required");
  if (!aligned16(q) || !aligned16(out) || (scores && !aligned16(scores)))
    return fail(TQ_ERR_ALIGNMENT, "q, out and scores must be 16-byte aligned");
  const int rows = Hq / Hkv * Tq;
  const bool vqjl = (layer->flags & TQ_LAYER_VALUE_QJL) != 0;
  if (vqjl ? !ref_decode_supports(layer->d, rows, true)
           : !mfma_decode_supports(layer->d, rows) && !ref_decode_supports(layer->d, rows, false))
    return fail(TQ_ERR_UNSUPPORTED, "(Hq/Hkv)*Tq too large for this head dimension");
  if ((int64_t)B * Hkv > 0x7FFFFFFF) return fail(TQ_ERR_UNSUPPORTED, "too many sequences");
  *plan = decode_plan(layer->d, layer->k_qjl, layer->flags & TQ_LAYER_DITHER, layer->flags & TQ_LAYER_VALUE_QJL, B,
                      Hq, Hkv, Tq, N);
  if (plan->nsplit > 65535) return fail(TQ_ERR_UNSUPPORTED, "too many key splits");
  return TQ_OK;
}

// Enqueues a checked decode call with its workspace at `workspace`.
tq_status launch_decode(const tq_layer* layer, const void* q, int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                        int32_t Tq, int64_t N, int32_t causal, const tq_cache* K, const tq_cache* V, float* out,
                        float* scores, const Plan& P, void* workspace, void* stream) {
  const BlobLayout BL = blob_layout(layer->d);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  DecodeArgs a{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Tq = Tq;
  a.N = N;
  a.cap = K->cap;
  a.causal = causal;
  a.d = layer->d;
  a.kb = layer->k_bits;
  a.vb = layer->v_bits;
  a.qjl = layer->k_qjl;
  a.R = blob_f(layer, BL.rot);
  a.S = blob_f(layer, BL.proj);
  a.cb = blob_f(layer, BL.codebook);
  a.kidx = K->idx;
  a.ksign = K->sign;
  a.knorm = K->norm;
  a.krnorm = K->rnorm;
  a.vidx = V->idx;
  a.vnorm = V->norm;
  a.out = out;
  a.scores = scores;
  a.q_rot = reinterpret_cast<float*>(ws + P.off_qrot);
  a.q_proj = reinterpret_cast<float*>(ws + P.off_qproj);
  a.part = reinterpret_cast<float*>(ws + P.off_part);
  a.nsplit = P.nsplit;
  a.waves = P.waves;
  a.wide = P.wide;
  a.keys_per_split = P.keys_per_split;
  a.dither = (layer->flags & TQ_LAYER_DITHER) != 0;
  a.vqjl = (layer->flags & TQ_LAYER_VALUE_QJL) != 0;
  a.vsign = V->sign;
  a.vrnorm = V->rnorm;
  a.kd0 = dither_stream_start(layer->seed, kDitherTagKeys);
  a.vd0 = dither_stream_start(layer->seed, kDitherTagValues);
  a.scales = blob_f(layer, BL.scales);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (P.mfma) {
    DecodeMfmaExtra x{};
    x.Rt = blob_f(layer, BL.rot_t);
    x.St = blob_f(layer, BL.proj_t);
    x.scales = blob_f(layer, BL.scales);
    x.rot_hi = blob_p(layer, BL.rot_hi);
    x.rot_lo = blob_p(layer, BL.rot_lo);
    x.proj_hi = blob_p(layer, BL.proj_hi);
    x.proj_lo = blob_p(layer, BL.proj_lo);
    return hip_status(launch_decode_mfma(a, x, st), "decode launch");
  }
  return hip_status(launch_decode_ref(a, st), "decode launch");
}
// Decode scratch of tq_attn_decode_static: a fixed device array, so that the
// call allocates nothing.  Host code must not use its name as an address (in
// host code it names a host-side stand-in): the device address is looked up
// once per device, with that device current, and kept in scratch_ptr.
constexpr size_t kScratchBytes = TQ_DECODE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device.
tq_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TQ_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress of the decode scratch");
    if (!p) return fail(TQ_ERR_HIP, "hipGetSymbolAddress returned no address for the decode scratch");
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return TQ_OK;
}
}  // namespace

tq_status fail(tq_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

}  // namespace tq

using namespace tq;

extern "C" {

int32_t tq_abi_version(void) { return TQ_ABI_VERSION; }

const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported";
    case TQ_ERR_ALIGNMENT: return "misaligned pointer";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    case TQ_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* tq_last_error(void) { return g_last_error.c_str(); }

size_t tq_layer_blob_bytes(int32_t d) { return supported_d(d) ? blob_layout(d).total : 0; }

tq_status tq_cache_bytes(const tq_layer* layer, int32_t which, int64_t seqs, int64_t cap,
                         size_t out[4]) {
  if (!layer || !out) return fail(TQ_ERR_INVALID_ARG, "layer and out are required");
  if (!supported_d(layer->d)) return fail(TQ_ERR_UNSUPPORTED, "d must be 64, 128 or 256");
  if (which != TQ_KEYS && which != TQ_VALUES) return fail(TQ_ERR_INVALID_ARG, "which must be TQ_KEYS or TQ_VALUES");
  if (seqs < 0 || cap <= 0 || cap % 8) return fail(TQ_ERR_INVALID_ARG, "need seqs >= 0 and cap a positive multiple of 8");
  const int bits = which == TQ_KEYS ? layer->k_bits : layer->v_bits;
  if (bits < 1 || bits > 4) return fail(TQ_ERR_INVALID_ARG, "bit widths must be 1..4");
  if (!seq_bytes_ok(layer->d, bits, cap))
    return fail(TQ_ERR_UNSUPPORTED, "cap * d * bits / 8 must stay below 2^31 - 2^20 bytes per sequence");
  const bool qjl = rows_qjl(layer, which);
  const size_t tokens = (size_t)seqs * (size_t)cap;
  out[0] = tokens * layer->d * bits / 8;
  out[1] = qjl ? tokens * layer->d / 8 : 0;
  out[2] = tokens * sizeof(float);
  out[3] = qjl ? tokens * sizeof(float) : 0;
  return TQ_OK;
}

tq_status tq_host_tables(int32_t d, int32_t rot, uint64_t seed, double* rotation,
                         double* projection) {
  if (!supported_d(d)) return fail(TQ_ERR_UNSUPPORTED, "d must be 64, 128 or 256");
  if (rot != TQ_ROT_HAAR && rot != TQ_ROT_HADAMARD) return fail(TQ_ERR_INVALID_ARG, "bad rot");
  if (rotation) make_rotation_f64(d, rot, seed, rotation);
  if (projection) make_projection_f64(d, seed, projection);
  return TQ_OK;
}

tq_status tq_get_codebook_law(int32_t d, int32_t bits, int32_t law, float* centroids, float* boundaries) {
  if (!supported_d(d)) return fail(TQ_ERR_UNSUPPORTED, "d must be 64, 128 or 256");
  if (bits < 1 || bits > 4) return fail(TQ_ERR_INVALID_ARG, "bits must be 1..4");
  if (law != TQ_LAW_GAUSSIAN && law != TQ_LAW_BETA) return fail(TQ_ERR_INVALID_ARG, "law must be TQ_LAW_GAUSSIAN or TQ_LAW_BETA");
  if (!centroids || !boundaries) return fail(TQ_ERR_INVALID_ARG, "outputs are required");
  if (law == TQ_LAW_BETA)
    lloyd_max_codebook_beta(bits, d, centroids, boundaries);
  else
    lloyd_max_codebook(bits, d, centroids, boundaries);
  return TQ_OK;
}

tq_status tq_get_codebook(int32_t d, int32_t bits, float* centroids, float* boundaries) {
  return tq_get_codebook_law(d, bits, TQ_LAW_GAUSSIAN, centroids, boundaries);
}

tq_status tq_make_layer(tq_layer* layer, int32_t d, int32_t rot, uint64_t seed, int32_t k_bits, int32_t k_qjl,
                        int32_t v_bits, int32_t flags, void* dev_blob, size_t blob_bytes, void* stream) {
  if (!layer) return fail(TQ_ERR_INVALID_ARG, "layer is NULL");
  if (!supported_d(d)) return fail(TQ_ERR_UNSUPPORTED, "d must be 64, 128 or 256");
  if (rot != TQ_ROT_HAAR && rot != TQ_ROT_HADAMARD) return fail(TQ_ERR_INVALID_ARG, "bad rot");
  if (k_bits < 1 || k_bits > 4 || v_bits < 1 || v_bits > 4)
    return fail(TQ_ERR_INVALID_ARG, "bit widths must be 1..4");
  if (k_qjl != 0 && k_qjl != 1) return fail(TQ_ERR_INVALID_ARG, "k_qjl must be 0 or 1");
  if (flags & ~kKnownLayerFlags) return fail(TQ_ERR_INVALID_ARG, "unknown layer flags");
  if (!dither_ok(flags, rot, k_qjl))
    return fail(TQ_ERR_INVALID_ARG, "TQ_LAYER_DITHER needs the Hadamard rotation and keys and values without QJL");
  if (!dev_blob) return fail(TQ_ERR_INVALID_ARG, "dev_blob is NULL");
  if (!aligned16(dev_blob)) return fail(TQ_ERR_ALIGNMENT, "dev_blob must be 16-byte aligned");
  const BlobLayout BL = blob_layout(d);
  if (blob_bytes < BL.total) return fail(TQ_ERR_INVALID_ARG, "blob_bytes < tq_layer_blob_bytes(d)");
  std::vector<unsigned char> image(BL.total);
  build_blob_image(d, rot, seed, k_bits, v_bits, flags, image.data());
  hipStream_t st = static_cast<hipStream_t>(stream);
  tq_status s = hip_status(hipMemcpyAsync(dev_blob, image.data(), BL.total, hipMemcpyHostToDevice, st),
                           "copy layer tables");
  if (s != TQ_OK) return s;
  s = hip_status(hipStreamSynchronize(st), "wait for layer tables");
  if (s != TQ_OK) return s;
  layer->d = d;
  layer->rot = rot;
  layer->k_bits = k_bits;
  layer->k_qjl = k_qjl;
  layer->v_bits = v_bits;
  layer->flags = flags;
  layer->seed = seed;
  layer->blob = dev_blob;
  layer->blob_bytes = blob_bytes;
  return TQ_OK;
}

tq_status tq_make_rotation(tq_layer* layer, int32_t d, int32_t rot, uint64_t seed, int32_t k_bits,
                           int32_t k_qjl, int32_t v_bits, void* dev_blob, size_t blob_bytes,
                           void* stream) {
  return tq_make_layer(layer, d, rot, seed, k_bits, k_qjl, v_bits, 0, dev_blob, blob_bytes, stream);
}

tq_status tq_quantize_kv(const tq_layer* layer, int32_t which, const void* x, int32_t dtype,
                         int64_t seqs, int64_t n, int64_t t0, const tq_cache* cache,
                         void* stream) {
  tq_status s = check_layer(layer);
  if (s != TQ_OK) return s;
  if (which != TQ_KEYS && which != TQ_VALUES) return fail(TQ_ERR_INVALID_ARG, "which must be TQ_KEYS or TQ_VALUES");
  if (dtype != TQ_F32 && dtype != TQ_F16) return fail(TQ_ERR_INVALID_ARG, "dtype must be TQ_F32 or TQ_F16");
  if ((s = check_cache(layer, which, cache, which == TQ_KEYS ? "K" : "V")) != TQ_OK) return s;
  if (seqs < 0 || n < 0 || t0 < 0) return fail(TQ_ERR_INVALID_ARG, "seqs, n and t0 must be >= 0");
  if (seqs > cache->seqs) return fail(TQ_ERR_INVALID_ARG, "seqs exceeds the cache's sequence count");
  if (t0 + n > cache->cap) return fail(TQ_ERR_INVALID_ARG, "t0 + n exceeds the cache capacity");
  if (seqs > 65535) return fail(TQ_ERR_UNSUPPORTED, "at most 65535 sequences per call");
  if (cache->cap > ((int64_t)1 << 24) || n * layer->d > ((int64_t)1 << 31) / 4)
    return fail(TQ_ERR_UNSUPPORTED, "at most 2^24 tokens per sequence");
  if (n > 0 && seqs > 0) {
    if (!x) return fail(TQ_ERR_INVALID_ARG, "x is NULL");
    if (!aligned16(x)) return fail(TQ_ERR_ALIGNMENT, "x must be 16-byte aligned");
  }
  const BlobLayout BL = blob_layout(layer->d);
  QuantizeArgs a{};
  a.x = x;
  a.dtype = dtype;
  a.seqs = seqs;
  a.n = n;
  a.t0 = t0;
  a.cap = cache->cap;
  a.d = layer->d;
  a.bits = which == TQ_KEYS ? layer->k_bits : layer->v_bits;
  a.qjl = rows_qjl(layer, which) ? 1 : 0;
  a.value_layout = which == TQ_VALUES;
  a.rot = layer->rot;
  a.dsign = blob_f(layer, BL.signs);
  a.R = blob_f(layer, BL.rot);
  a.SR = blob_f(layer, BL.projr);
  a.cent = blob_f(layer, BL.codebook) + (which == TQ_KEYS ? 0 : 2 * kMaxLevels);
  a.bnd = a.cent + kMaxLevels;
  a.rot_hi = blob_p(layer, BL.rot_hi);
  a.rot_lo = blob_p(layer, BL.rot_lo);
  a.projr_hi = blob_p(layer, BL.projr_hi);
  a.projr_lo = blob_p(layer, BL.projr_lo);
  a.idx = cache->idx;
  a.sign = cache->sign;
  a.norm = cache->norm;
  a.rnorm = cache->rnorm;
  a.dither = (layer->flags & TQ_LAYER_DITHER) != 0;
  a.dither_s0 = dither_stream_start(layer->seed, which == TQ_KEYS ? kDitherTagKeys : kDitherTagValues);
  a.dither_w = blob_f(layer, BL.scales) + (which == TQ_KEYS ? 4 : 5);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.dither && !fwht_quantize_supports(a.d, a.rot, a.qjl))
    return fail(TQ_ERR_UNSUPPORTED, "the dithered variant needs the transform quantizer");
  // Values with QJL: only the reference kernel writes sign rows for the value layout.
  if (a.value_layout && a.qjl) return hip_status(launch_quantize_ref(a, st), "quantize launch");
  if (fwht_quantize_supports(a.d, a.rot, a.qjl)) return hip_status(launch_quantize_fwht(a, st), "quantize launch");
  if (mfma_quantize_supports(a.d, a.dtype)) return hip_status(launch_quantize_mfma(a, st), "quantize launch");
  return hip_status(launch_quantize_ref(a, st), "quantize launch");
}

size_t tq_decode_workspace_bytes(const tq_layer* layer, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t Tq, int64_t N) {
  if (!layer || !supported_d(layer->d) || B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || N < 1) return 0;
  return decode_plan(layer->d, layer->k_qjl, layer->flags & TQ_LAYER_DITHER, layer->flags & TQ_LAYER_VALUE_QJL, B,
                     Hq, Hkv, Tq, N).total;
}

tq_status tq_attn_decode(const tq_layer* layer, const void* q, int32_t q_dtype, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t Tq, int64_t N, int32_t causal,
                         const tq_cache* K, const tq_cache* V, float* out, float* scores,
                         void* workspace, size_t workspace_bytes, void* stream) {
  Plan P{};
  tq_status s = check_decode(layer, q, q_dtype, B, Hq, Hkv, Tq, N, causal, K, V, out, scores, &P);
  if (s != TQ_OK) return s;
  if (!workspace) return fail(TQ_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(TQ_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < P.total) return fail(TQ_ERR_WORKSPACE, "workspace smaller than tq_decode_workspace_bytes");
  return launch_decode(layer, q, q_dtype, B, Hq, Hkv, Tq, N, causal, K, V, out, scores, P, workspace, stream);
}

tq_status tq_attn_decode_static(const tq_layer* layer, const void* q, int32_t q_dtype, int32_t B,
                                int32_t Hq, int32_t Hkv, int32_t Tq, int64_t N, int32_t causal,
                                const tq_cache* K, const tq_cache* V, float* out, float* scores,
                                void* stream) {
  Plan P{};
  tq_status s = check_decode(layer, q, q_dtype, B, Hq, Hkv, Tq, N, causal, K, V, out, scores, &P);
  if (s != TQ_OK) return s;
  if (P.total > kScratchBytes)
    return fail(TQ_ERR_WORKSPACE, "this shape needs " + std::to_string(P.total) +
                                      " bytes of decode scratch; tq_attn_decode_static holds " +
                                      std::to_string(kScratchBytes) + " (call tq_attn_decode with a workspace)");
  void* ws = nullptr;
  if ((s = scratch_for_current_device(&ws)) != TQ_OK) return s;
  return launch_decode(layer, q, q_dtype, B, Hq, Hkv, Tq, N, causal, K, V, out, scores, P, ws, stream);
}

tq_status tq_dequantize(const tq_layer* layer, int32_t which, const tq_cache* cache, int64_t n,
                        void* out, int32_t out_dtype, void* stream) {
  tq_status s = check_dequantize(layer, which, cache, n, out, out_dtype, false);
  if (s != TQ_OK) return s;
  return hip_status(launch_dequant(dequant_args(layer, which, cache, n, out, out_dtype),
                                        static_cast<hipStream_t>(stream)),
                    "dequantize launch");
}

tq_status tq_dequantize_prod(const tq_layer* layer, int32_t which, const tq_cache* cache, int64_t n,
                             void* out, int32_t out_dtype, void* stream) {
  tq_status s = check_dequantize(layer, which, cache, n, out, out_dtype, true);
  if (s != TQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const BlobLayout BL = blob_layout(layer->d);
  DequantArgs a = dequant_args(layer, which, cache, n, out, out_dtype);
  if (which == TQ_KEYS && layer->rot != TQ_ROT_HADAMARD && layer->d <= 128 && !a.dither) {
    // One pass: the matrix-core dequantize adds the QJL term before it stores.
    a.qjl = 1;
    a.sign = cache->sign;
    a.rnorm = cache->rnorm;
    a.St = blob_f(layer, BL.proj_t);
    return hip_status(launch_dequant(a, st), "dequantize launch");
  }
  s = hip_status(launch_dequant(a, st), "dequantize launch");
  if (s != TQ_OK) return s;
  DequantQjlArgs q{};
  q.sign = cache->sign;
  q.norm = cache->norm;
  q.rnorm = cache->rnorm;
  q.seqs = cache->seqs;
  q.n = n;
  q.cap = cache->cap;
  q.d = layer->d;
  q.St = blob_f(layer, BL.proj_t);
  q.out = out;
  q.out_dtype = out_dtype;
  return hip_status(launch_dequant_qjl(q, st), "dequantize QJL launch");
}

}  // extern "C"
