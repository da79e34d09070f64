// Dequantisation kernel of libtq and tq_dequantize: dense float32
// reconstruction xhat = (n / d) D H D c[code] (+ the QJL residual of keys),
// used to check the codec ("TurboMOQ", Quick Start: decompress).
#include "tq_device.h"

namespace tq {
namespace dev {
namespace {

// -------------------------------------------------------------- dequantize
struct DequantArgs {
  const uint64_t* pages;
  int n_kv_heads, max_pages;
  const char* pool;
  uint64_t pool_bytes;
  const uint32_t* sign_mask;
  const float* table;
  const float* qjl_s;
  int which, add_qjl, tok0, ntok, page0;
  int polar;   // the part is PolarQuant-coded: code pairs (radius, angle)
  float* out;
};

// Code n of stream s of a block staged in LDS (word-interleaved layout).
__device__ __forceinline__ uint32_t stream_code(const uint32_t* blk, int b, int s, int n) {
  const int pos = n * b, dw = pos >> 5, sh = pos & 31;
  auto dword = [&](int d) { return blk[((d >> 2) * 64 + s) * 4 + (d & 3)]; };
  uint32_t v = dword(dw) >> sh;
  if (sh + b > 32) v |= dword(dw + 1) << (32 - sh);
  return v & ((1u << b) - 1u);
}

__global__ __launch_bounds__(64) void dequant_kernel(DequantArgs a, const float* __restrict__ qjl_s) {
  __shared__ uint32_t blk[2048];  // up to an 8-bit block (8 KB)
  __shared__ float cent[256];
  __shared__ float2 pair[256];
  const int lane = threadIdx.x;
  const int pg = a.page0 + blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const uint64_t desc = a.pages[((size_t)b * a.n_kv_heads + h) * a.max_pages + pg];
  const int t = pg * PT + lane;
  const bool in_range = t >= a.tok0 && t < a.tok0 + a.ntok;
  float* dst = a.out + (((size_t)b * a.n_kv_heads + h) * a.ntok + (size_t)(t - a.tok0)) * D;
  const PageDesc pd = read_desc(desc);
  const int kb = pd.kb, vb = pd.vb;
  const bool qjl = pd.qjl;
  const uint64_t off = pd.off;
  const bool bad = !pd.present || off + page_size_dev(kb, vb, qjl) > a.pool_bytes ||
                   (kb == 0 && (vb != 0 || qjl)) || kb > 8 || (kb > 0 && (vb < 1 || vb > 8)) ||
                   (a.polar && (a.which == 0 ? kb : vb) > 4);
  if (bad) {
    if (in_range)
      for (int j = 0; j < D; ++j) dst[j] = __builtin_nanf("");
    return;
  }
  const char* page = a.pool + off;
  if (kb == 0) {
    if (!in_range) return;
    const __half* row = reinterpret_cast<const __half*>(page + a.which * PT * D * 2) + (size_t)lane * D;
    for (int j = 0; j < D; ++j) dst[j] = __half2float(row[j]);
    return;
  }
  const int B = a.which == 0 ? kb : vb;
  const char* blk_src = a.which == 0 ? page : page + 1024 * kb + 256 + (qjl ? 1280 : 0);
  const float norm = reinterpret_cast<const float*>(blk_src + 1024 * B)[lane];
  for (int i = lane; i < 256 * B; i += 64) blk[i] = reinterpret_cast<const uint32_t*>(blk_src)[i];
  for (int i = lane; i < (1 << B); i += 64) cent[i] = a.table[centroid_offset(B) + i];
  if (a.polar) {
    const float2* pt = reinterpret_cast<const float2*>(a.table + kPairOffset) + pair_offset_host(B);
    for (int i = lane; i < (1 << (2 * B)); i += 64) pair[i] = pt[i];
  }
  __syncthreads();
  if (!in_range) return;
  uint32_t m[4];
  for (int w = 0; w < 4; ++w) m[w] = a.sign_mask[w];
  float x[D];
  // code of coordinate j of this lane's token
  auto code_of = [&](int j) {
    if (a.which == 0) return stream_code(blk, B, lane, j);
    // V: coordinate j is in stream n + 32 P at position 2 t + (j & 1) (the
    // inverse of v_stream_coord)
    const int n = ((j >> 1) & 3) | (((j >> 6) & 1) << 2) | (((j >> 3) & 3) << 3), P = (j >> 5) & 1;
    return stream_code(blk, B, n + 32 * P, 2 * lane + (j & 1));
  };
  if (a.polar) {
    // pair i: radius code at coordinate 2i, angle code at 2i + 1
#pragma clang loop unroll(full)
    for (int i = 0; i < D / 2; ++i) {
      const float2 v = pair[checked(code_of(2 * i) | (code_of(2 * i + 1) << B), 1 << (2 * B), kCheckDecodeTable)];
      x[2 * i] = v.x;
      x[2 * i + 1] = v.y;
    }
  } else {
#pragma clang loop unroll(full)
    for (int j = 0; j < D; ++j) x[j] = cent[checked(code_of(j), 1 << B, kCheckDecodeTable)];
  }
  // xhat = (n / sqrt(d)) R c = (n / d) D H D c
#pragma clang loop unroll(full)
  for (int j = 0; j < D; ++j) x[j] = flip_if(x[j], dsign(m, j));
  fwht128(x);
  const float sc = norm * (1.0f / D);
#pragma clang loop unroll(full)
  for (int j = 0; j < D; ++j) x[j] = flip_if(x[j], dsign(m, j)) * sc;
  if (a.which == 0 && qjl && a.add_qjl && qjl_s) {
    const char* qb = page + 1024 * kb + 256;
    const uint4 zw4 = reinterpret_cast<const uint4*>(qb)[lane];
    const uint32_t zw[4] = {zw4.x, zw4.y, zw4.z, zw4.w};
    const float gamma = reinterpret_cast<const float*>(qb + 1024)[lane];
    const float coef = kSqrtHalfPi / TQ_JL_DIM * gamma;
    for (int i = 0; i < TQ_JL_DIM; ++i) {
      const float zi = ((zw[i >> 5] >> (i & 31)) & 1u) ? coef : -coef;
      const float* srow = qjl_s + (size_t)i * D;
#pragma clang loop unroll(full)
      for (int j = 0; j < D; ++j) x[j] = fmaf(zi, srow[j], x[j]);
    }
  }
  float4* d4 = reinterpret_cast<float4*>(dst);
#pragma clang loop unroll(full)
  for (int c = 0; c < D / 4; ++c) d4[c] = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
}


}  // namespace
}  // namespace dev
}  // namespace tq

using namespace tq;
using namespace tq::dev;

int tq::check_word_dequant(uint32_t* out, bool reset) { return read_check_word(out, reset); }

extern "C" {

int tq_dequantize(const tq_layer* layer, const tq_cache* cache, int which, int add_qjl, int tok0,
                  int ntok, float* out, void* stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (which != 0 && which != 1) return fail(TQ_ERR_INVALID_ARG, "which must be 0 (K) or 1 (V)");
  if (!out) return fail(TQ_ERR_INVALID_ARG, "null output");
  if (!aligned16(out)) return fail(TQ_ERR_ALIGNMENT, "output must be 16-byte aligned");
  if (tok0 < 0 || ntok < 1 || (int64_t)tok0 + ntok > (int64_t)cache->max_pages * TQ_PAGE_TOKENS)
    return fail(TQ_ERR_INVALID_ARG, "bad token range");
  DequantArgs a;
  a.pages = cache->pages;
  a.n_kv_heads = cache->n_kv_heads;
  a.max_pages = cache->max_pages;
  a.pool = reinterpret_cast<const char*>(cache->pool);
  a.pool_bytes = cache->pool_bytes;
  a.sign_mask = layer->sign_mask;
  a.table = which == 0 ? layer->k_table : layer->v_table;
  a.qjl_s = layer->qjl_s;
  a.which = which;
  a.add_qjl = add_qjl;
  a.tok0 = tok0;
  a.ntok = ntok;
  a.page0 = tok0 / TQ_PAGE_TOKENS;
  a.polar = (which == 0 ? layer->k_codebook : layer->v_codebook) == TQ_CODEBOOK_POLAR;
  a.out = out;
  const int last_page = (tok0 + ntok - 1) / TQ_PAGE_TOKENS;
  dim3 grid(last_page - a.page0 + 1, cache->n_kv_heads, cache->n_sessions);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(64), 0, (hipStream_t)stream, a, layer->qjl_s);
  return launch_status("dequantize");
}

}  // extern "C"
