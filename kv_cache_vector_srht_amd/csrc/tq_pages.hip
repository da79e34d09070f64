// Page maintenance kernels of libtq for gfx950: the decode loop's append
// (tq_append_kv) and re-tiering (tq_retier_pages).
//
// Append ("TurboQuant-MLX v2.0", What's New > FP16 Attention Sinks and Dynamic
// Chunk Buffering): new tokens go to an fp16 tail page, packed in place when
// its 64th token arrives.  Re-tiering ("TurboMOQ", Progressive temporal
// tiering; Attention-weighted tier demotion): pages move to narrower formats
// in place, through a code-to-code table, or from fp16 into a packed format.
#include <algorithm>

#include "tq_device.h"
#include "tq_token_encoder.h"

namespace tq {
namespace dev {
namespace {

// ------------------------------------------------------- decode-loop append
struct AppendArgs {
  int k_polar, v_polar;   // PolarQuant parts (at most 4 bits wide)
  const void* k;
  const void* v;
  int dtype;
  int64_t sb, sh;
  int32_t* err;
  uint64_t* pages;
  int n_kv_heads, max_pages;
  const int32_t* n_tokens;
  char* pool;
  uint64_t pool_bytes;
  const uint32_t* sign_mask;
  const float* k_table;
  const float* v_table;
  const float* qjl_s;
};

// One wavefront per (KV head, session): writes the new token's rows into its
// fp16 or pending page; when a pending page receives its 64th token, encodes
// the page in place with the per-token encoder (keys, then values; every lane
// loads its row before any lane stores, and the key part ends below the value
// rows) and clears the pending bit.
// POLAR: the instantiation for layers with PolarQuant parts (the plain one has
// no polar code, which keeps its registers).
template <bool POLAR>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  __shared__ float lds_thr[256];
  __shared__ float lds_cent[256];
  __shared__ float2 lds_pair[256];
  __shared__ uint32_t lds_rows[PT * kEncodeRowBytes / 4];
  const int lane = threadIdx.x, h = blockIdx.x, b = blockIdx.y;
  const int t = a.n_tokens[b];
  if (t < 0 || t >= a.max_pages * PT) {
    if (lane == 0) raise_flag(a.err, 16);
    return;
  }
  const int r = t & (PT - 1);
  uint64_t* dp = a.pages + ((size_t)b * a.n_kv_heads + h) * a.max_pages + t / PT;
  const uint64_t desc = *dp;
  if (!(desc & TQ_PAGE_PRESENT)) {
    if (lane == 0) raise_flag(a.err, 2);
    return;
  }
  const bool pending = (desc & TQ_PAGE_PENDING) != 0;
  const int kb = (int)((desc >> 48) & 15), vb = (int)((desc >> 52) & 15);
  const bool qjl = (desc & TQ_PAGE_QJL) != 0;
  const uint64_t off = desc & TQ_PAGE_OFFSET_MASK;
  if (!pending && kb != 0) {
    if (lane == 0) raise_flag(a.err, 32);
    return;
  }
  const int tk = a.k_polar ? polar_shift_of(a.k_table) : 0, tv = a.v_polar ? polar_shift_of(a.v_table) : 0;
  const bool bad_target = pending && (kb < 1 || kb > 8 || vb < 1 || vb > 8 || (qjl && !a.qjl_s) ||
                                      (a.k_polar && !polar_width_ok(kb, tk)) ||
                                      (a.v_polar && !polar_width_ok(vb, tv)));
  if (bad_target || off + page_size_dev(0, 0, false) > a.pool_bytes) {
    if (lane == 0) raise_flag(a.err, 4);
    return;
  }
  char* page = a.pool + off;
  if (lane < 32) {
    const int part = lane >> 4, c8 = (lane & 15) * 8;
    const void* src = part == 0 ? a.k : a.v;
    const size_t ee = (size_t)b * a.sb + (size_t)h * a.sh + c8;
    uint4 out;
    if (a.dtype == TQ_DTYPE_F16) {
      out = *reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(src) + ee);
    } else {
      const float4 f0 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + ee);
      const float4 f1 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + ee + 4);
      __half2 h0 = __floats2half2_rn(f0.x, f0.y), h1 = __floats2half2_rn(f0.z, f0.w);
      __half2 h2 = __floats2half2_rn(f1.x, f1.y), h3 = __floats2half2_rn(f1.z, f1.w);
      out = make_uint4(*reinterpret_cast<uint32_t*>(&h0), *reinterpret_cast<uint32_t*>(&h1),
                       *reinterpret_cast<uint32_t*>(&h2), *reinterpret_cast<uint32_t*>(&h3));
    }
    *reinterpret_cast<uint4*>(page + part * PT * D * 2 + ((size_t)r * D + c8) * 2) = out;
  }
  if (!pending || r != PT - 1) return;
  // the page is complete: make the row just written visible to every lane
  __threadfence();
  __syncthreads();
  uint32_t m[4];
#pragma clang loop unroll(full)
  for (int w = 0; w < 4; ++w) m[w] = a.sign_mask[w];
  for (int part = 0; part < 2; ++part) {
    const int B = part == 0 ? kb : vb;
    const float* table = part == 0 ? a.k_table : a.v_table;
    const bool polar = POLAR && (part == 0 ? a.k_polar : a.v_polar);
    const int shift = part == 0 ? tk : tv;
    stage_token_tables(table, B, polar, shift, lane, 64, lds_thr, lds_cent, lds_pair);
    float x[D];
    load_row(page + part * PT * D * 2, TQ_DTYPE_F16, (size_t)lane * D, x);
    __syncthreads();
    char* part_base = part == 0 ? page : page + 1024 * kb + 256 + (qjl ? 1280 : 0);
    float n = 0.f;
    if (part == 0) {
      switch (B) {
        case 1: n = encode_packed<0, 1>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 2: n = encode_packed<0, 2>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 3: n = encode_packed<0, 3>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 4: n = encode_packed<0, 4>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 5: n = encode_packed<0, 5>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 6: n = encode_packed<0, 6>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 7: n = encode_packed<0, 7>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        default: n = encode_packed<0, 8>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
      }
      if (qjl) qjl_sketch(a.qjl_s, part_base + 1024 * B + 256, lane, x, m, n);
    } else {
      switch (B) {
        case 1: n = encode_packed<1, 1>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 2: n = encode_packed<1, 2>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 3: n = encode_packed<1, 3>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 4: n = encode_packed<1, 4>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 5: n = encode_packed<1, 5>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 6: n = encode_packed<1, 6>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        case 7: n = encode_packed<1, 7>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
        default: n = encode_packed<1, 8>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
      }
    }
    __syncthreads();
  }
  if (lane == 0) *dp = desc & ~TQ_PAGE_PENDING;
}

// n_tokens[b] += 1 for every session, after the append above.
__global__ __launch_bounds__(256) void advance_kernel(int32_t* n_tokens, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) n_tokens[i] += 1;
}

// ------------------------------------------------------------- re-tiering
// Workgroups of the re-tiering launches (one wave each, striding over the
// list): eight per CU of MI355X, as many as the packed instance's LDS allows.
constexpr int kRetierBlocks = 2048;

struct RetierArgs {
  int k_polar, v_polar;   // PolarQuant parts (at most 4 bits wide)
  const int64_t* index;
  const uint64_t* new_desc;
  int n;
  int sources;        // TQ_RETIER_FROM_* bits of the launched instances
  int raise_errors;   // this launch raises the error flags
  int32_t* err;
  uint64_t* pages;
  int64_t n_entries;
  char* pool;
  uint64_t pool_bytes;
  const uint32_t* sign_mask;
  const float* k_table;
  const float* v_table;
  const float* qjl_s;
};

// Stream `lane` of a B-bit code block (word w at (w * 64 + lane) * 16),
// unpacked and mapped through `map` into this lane's LDS row of 128 bytes.
template <int B>
__device__ __forceinline__ void unpack_mapped(const uint4* __restrict__ blk, int lane, const uint8_t* map,
                                              uint4* row) {
  uint32_t s[4 * B];
#pragma clang loop unroll(full)
  for (int i = 0; i < B; ++i) {
    const uint4 w = blk[i * 64 + lane];
    s[4 * i] = w.x;
    s[4 * i + 1] = w.y;
    s[4 * i + 2] = w.z;
    s[4 * i + 3] = w.w;
  }
  // up to 4 bits the map fits one 64-bit word as nibbles: a shift instead of
  // an LDS read per code
  uint64_t mw = 0;
  if constexpr (B <= 4) {
#pragma clang loop unroll(full)
    for (int c = 0; c < (1 << B); ++c) mw |= (uint64_t)map[c] << (4 * c);
  }
#pragma clang loop unroll(full)
  for (int i = 0; i < D / 16; ++i) {
    uint32_t o[4];
#pragma clang loop unroll(full)
    for (int k = 0; k < 4; ++k) {
      uint32_t v = 0;
#pragma clang loop unroll(full)
      for (int e = 0; e < 4; ++e) {
        const uint32_t c = bits_at(s, (16 * i + 4 * k + e) * B, B);
        const uint32_t m = B <= 4 ? (uint32_t)(mw >> (4 * c)) & 15u : (uint32_t)map[checked((int)c, 1 << B, kCheckPages)];
        v |= m << (8 * e);
      }
      o[k] = v;
    }
    row[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// The inverse: this lane's row of byte codes (each < 2^B) packed into stream
// `lane` of a B-bit block.
template <int B>
__device__ __forceinline__ void pack_row(const uint4* row, int lane, uint4* __restrict__ blk) {
  uint32_t s[4 * B];
#pragma clang loop unroll(full)
  for (int i = 0; i < 4 * B; ++i) s[i] = 0;
#pragma clang loop unroll(full)
  for (int i = 0; i < D / 16; ++i) {
    const uint4 r = row[i];
    const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma clang loop unroll(full)
    for (int e = 0; e < 16; ++e) {
      const uint32_t c = (rw[e >> 2] >> (8 * (e & 3))) & 0xffu;
      const int pos = (16 * i + e) * B, wi = pos >> 5, sh = pos & 31;
      s[wi] |= c << sh;
      if (sh + B > 32) s[wi + 1] |= c >> (32 - sh);
    }
  }
#pragma clang loop unroll(full)
  for (int i = 0; i < B; ++i) blk[i * 64 + lane] = make_uint4(s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
}

__device__ __forceinline__ void unpack_mapped_any(int b, const uint4* blk, int lane, const uint8_t* map,
                                                  uint4* row) {
  switch (b) {
    case 1: unpack_mapped<1>(blk, lane, map, row); break;
    case 2: unpack_mapped<2>(blk, lane, map, row); break;
    case 3: unpack_mapped<3>(blk, lane, map, row); break;
    case 4: unpack_mapped<4>(blk, lane, map, row); break;
    case 5: unpack_mapped<5>(blk, lane, map, row); break;
    case 6: unpack_mapped<6>(blk, lane, map, row); break;
    case 7: unpack_mapped<7>(blk, lane, map, row); break;
    default: unpack_mapped<8>(blk, lane, map, row); break;
  }
}

__device__ __forceinline__ void pack_row_any(int b, const uint4* row, int lane, uint4* blk) {
  switch (b) {
    case 1: pack_row<1>(row, lane, blk); break;
    case 2: pack_row<2>(row, lane, blk); break;
    case 3: pack_row<3>(row, lane, blk); break;
    case 4: pack_row<4>(row, lane, blk); break;
    case 5: pack_row<5>(row, lane, blk); break;
    case 6: pack_row<6>(row, lane, blk); break;
    case 7: pack_row<7>(row, lane, blk); break;
    default: pack_row<8>(row, lane, blk); break;
  }
}

// map[c] = the new-width code of old centroid c: the number of new-width
// boundaries at or below it (the quantiser's own rule, applied to the value
// the old code stands for).
__device__ __forceinline__ void build_code_map(const float* table, int ob, int nb, uint8_t* map, int lane) {
  const int nt = (1 << nb) - 1;
  for (int c = lane; c < (1 << ob); c += 64) {
    const float u = table[centroid_offset(ob) + c];
    int n = 0;
    for (int j = 0; j < nt; ++j) n += table[boundary_offset(nb) + j] <= u ? 1 : 0;
    map[c] = (uint8_t)n;
  }
}

// The checks of one listed page: 0 when it can be re-tiered, else the error
// flag it raises.
__device__ __forceinline__ int retier_check(const RetierArgs& a, int64_t idx, uint64_t od, uint64_t nd) {
  if (idx < 0 || idx >= a.n_entries) return 16;
  if (!(od & TQ_PAGE_PRESENT) || !(nd & TQ_PAGE_PRESENT)) return 2;
  const int kb = (int)((od >> 48) & 15), vb = (int)((od >> 52) & 15);
  const int nkb = (int)((nd >> 48) & 15), nvb = (int)((nd >> 52) & 15);
  const bool oq = (od & TQ_PAGE_QJL) != 0, nq = (nd & TQ_PAGE_QJL) != 0;
  const uint64_t ooff = od & TQ_PAGE_OFFSET_MASK, noff = nd & TQ_PAGE_OFFSET_MASK;
  const bool bad_old = kb == 0 ? (vb != 0 || oq) : (kb > 8 || vb < 1 || vb > 8);
  const bool bad_new = nkb < 1 || nkb > 8 || nvb < 1 || nvb > 8;
  const size_t osz = page_size_dev(kb, vb, oq), nsz = page_size_dev(nkb, nvb, nq);
  if (bad_old || bad_new || ooff + osz > a.pool_bytes || noff + nsz > a.pool_bytes ||
      (noff != ooff && noff < ooff + osz && ooff < noff + nsz))
    return 4;
  if (((od | nd) & TQ_PAGE_PENDING) || (kb != 0 && (oq || nq || nkb > kb || nvb > vb))) return 64;
  // PolarQuant: no code-to-code map (pairs of codes); fp16 sources encode at
  // most 4 bits wide
  if (kb != 0 && (a.k_polar || a.v_polar)) return 64;
  if ((a.k_polar && !polar_width_ok(nkb, polar_shift_of(a.k_table))) ||
      (a.v_polar && !polar_width_ok(nvb, polar_shift_of(a.v_table))))
    return 4;
  if (nq && !a.qjl_s) return 8;
  return 0;
}

// One wavefront per workgroup, striding over the listed pages; FROM_FP16
// selects the pages of one source kind, the other instance handles the rest.
// The first instance launched raises the error flags of every listed page
// (the second finds the same errors on the unchanged descriptors and skips
// them silently); a page of a source kind the launch leaves out counts as an
// unsupported change.  A packed page (no QJL) is re-coded stream by stream to
// narrower widths, keeping its norms; an fp16 page is encoded with the
// per-token encoder.  Every lane loads the whole of its part of the old page
// before any lane stores, so the new page may take the old slot.
template <bool FROM_FP16, bool POLAR>
__global__ __launch_bounds__(64) void retier_kernel(RetierArgs a) {
  __shared__ float lds_thr[FROM_FP16 ? 256 : 1];
  __shared__ float lds_cent[FROM_FP16 ? 256 : 1];
  __shared__ float2 lds_pair[FROM_FP16 ? 256 : 1];
  __shared__ uint32_t lds_rows[(FROM_FP16 ? 1 : 2) * PT * kEncodeRowBytes / 4];
  __shared__ uint8_t lds_map[2][256];
  __shared__ float lds_norm[2][FROM_FP16 ? 1 : PT];
  const int lane = threadIdx.x;
  for (int item = blockIdx.x; item < a.n; item += gridDim.x) {
    const int64_t idx = a.index[item];
    const bool in_table = idx >= 0 && idx < a.n_entries;
    uint64_t* dp = a.pages + (in_table ? idx : 0);
    const uint64_t od = in_table ? *dp : 0, nd = a.new_desc[item];
    int e = retier_check(a, idx, od, nd);
    const int kb = (int)((od >> 48) & 15), vb = (int)((od >> 52) & 15);
    if (!e && !(a.sources & (kb == 0 ? TQ_RETIER_FROM_FP16 : TQ_RETIER_FROM_PACKED))) e = 64;
    if (e) {
      if (a.raise_errors && lane == 0) raise_flag(a.err, e);
      continue;
    }
    const int nkb = (int)((nd >> 48) & 15), nvb = (int)((nd >> 52) & 15);
    const bool nq = (nd & TQ_PAGE_QJL) != 0;
    if ((kb == 0) != FROM_FP16) continue;
    const char* src = a.pool + (od & TQ_PAGE_OFFSET_MASK);
    char* dst = a.pool + (nd & TQ_PAGE_OFFSET_MASK);
    if constexpr (FROM_FP16) {
      uint32_t m[4];
#pragma clang loop unroll(full)
      for (int w = 0; w < 4; ++w) m[w] = a.sign_mask[w];
      for (int part = 0; part < 2; ++part) {
        const int B = part == 0 ? nkb : nvb;
        const float* table = part == 0 ? a.k_table : a.v_table;
        const bool polar = POLAR && (part == 0 ? a.k_polar : a.v_polar);
        const int shift = polar ? polar_shift_of(table) : 0;
        stage_token_tables(table, B, polar, shift, lane, 64, lds_thr, lds_cent, lds_pair);
        float x[D];
        load_row(src + part * PT * D * 2, TQ_DTYPE_F16, (size_t)lane * D, x);
        // the key part ends below the value rows, so in place the values are
        // still intact when they are loaded here
        __syncthreads();
        char* part_base = part == 0 ? dst : dst + 1024 * nkb + 256 + (nq ? 1280 : 0);
        float n = 0.f;
        if (part == 0) {
          switch (B) {
            case 1: n = encode_packed<0, 1>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 2: n = encode_packed<0, 2>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 3: n = encode_packed<0, 3>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 4: n = encode_packed<0, 4>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 5: n = encode_packed<0, 5>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 6: n = encode_packed<0, 6>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 7: n = encode_packed<0, 7>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            default: n = encode_packed<0, 8>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
          }
          if (nq) qjl_sketch(a.qjl_s, part_base + 1024 * B + 256, lane, x, m, n);
        } else {
          switch (B) {
            case 1: n = encode_packed<1, 1>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 2: n = encode_packed<1, 2>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 3: n = encode_packed<1, 3>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 4: n = encode_packed<1, 4>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 5: n = encode_packed<1, 5>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 6: n = encode_packed<1, 6>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            case 7: n = encode_packed<1, 7>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
            default: n = encode_packed<1, 8>(part_base, lane, x, m, lds_thr, lds_cent, lds_rows, polar, lds_pair, shift); break;
          }
        }
        __syncthreads();
      }
    } else {
      build_code_map(a.k_table, kb, nkb, lds_map[0], lane);
      build_code_map(a.v_table, vb, nvb, lds_map[1], lane);
      __syncthreads();
      // every load of the old page, then (after the barrier) every store
      uint4* krow = reinterpret_cast<uint4*>(reinterpret_cast<char*>(lds_rows) + lane * kEncodeRowBytes);
      uint4* vrow = reinterpret_cast<uint4*>(reinterpret_cast<char*>(lds_rows) + (PT + lane) * kEncodeRowBytes);
      const char* ov = src + 1024 * kb + 256;
      unpack_mapped_any(kb, reinterpret_cast<const uint4*>(src), lane, lds_map[0], krow);
      unpack_mapped_any(vb, reinterpret_cast<const uint4*>(ov), lane, lds_map[1], vrow);
      // the norms pass through LDS too, so that every load of the old page has
      // returned before the first store (the barrier of a one-wave block does
      // not wait for vector memory)
      lds_norm[0][lane] = reinterpret_cast<const float*>(src + 1024 * kb)[lane];
      lds_norm[1][lane] = reinterpret_cast<const float*>(ov + 1024 * vb)[lane];
      __syncthreads();
      char* nv = dst + 1024 * nkb + 256;
      pack_row_any(nkb, krow, lane, reinterpret_cast<uint4*>(dst));
      pack_row_any(nvb, vrow, lane, reinterpret_cast<uint4*>(nv));
      reinterpret_cast<float*>(dst + 1024 * nkb)[lane] = lds_norm[0][lane];
      reinterpret_cast<float*>(nv + 1024 * nvb)[lane] = lds_norm[1][lane];
    }
    if (lane == 0) *dp = nd;
    __syncthreads();   // LDS is reused by the next page
  }
}

}  // namespace
}  // namespace dev
}  // namespace tq

using namespace tq;
using namespace tq::dev;

int tq::check_word_pages(uint32_t* out, bool reset) { return read_check_word(out, reset); }

extern "C" {

int tq_append_kv(const tq_layer* layer, const tq_cache* cache, const tq_token_input* in, void* stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!in || !in->k || !in->v) return fail(TQ_ERR_INVALID_ARG, "null input");
  if (in->dtype != TQ_DTYPE_F16 && in->dtype != TQ_DTYPE_F32)
    return fail(TQ_ERR_INVALID_ARG, "unknown input dtype %d", in->dtype);
  if (in->stride_b < 0 || in->stride_h < 0) return fail(TQ_ERR_INVALID_ARG, "negative stride");
  const int esz = in->dtype == TQ_DTYPE_F16 ? 2 : 4;
  if (!aligned16(in->k) || !aligned16(in->v) || (in->stride_b * esz) % 16 || (in->stride_h * esz) % 16)
    return fail(TQ_ERR_ALIGNMENT, "input rows must be 16-byte aligned");
  if (((uintptr_t)in->error_flags & 3) != 0) return fail(TQ_ERR_ALIGNMENT, "error_flags misaligned");
  AppendArgs a;
  a.k = in->k;
  a.v = in->v;
  a.dtype = in->dtype;
  a.sb = in->stride_b;
  a.sh = in->stride_h;
  a.err = in->error_flags;
  a.pages = const_cast<uint64_t*>(cache->pages);
  a.n_kv_heads = cache->n_kv_heads;
  a.max_pages = cache->max_pages;
  a.n_tokens = cache->n_tokens;
  a.pool = reinterpret_cast<char*>(cache->pool);
  a.pool_bytes = cache->pool_bytes;
  a.sign_mask = layer->sign_mask;
  a.k_table = layer->k_table;
  a.v_table = layer->v_table;
  a.qjl_s = layer->qjl_s;
  a.k_polar = layer->k_codebook == TQ_CODEBOOK_POLAR;
  a.v_polar = layer->v_codebook == TQ_CODEBOOK_POLAR;
  hipStream_t s = (hipStream_t)stream;
  if (a.k_polar || a.v_polar)
    hipLaunchKernelGGL(append_kernel<true>, dim3(cache->n_kv_heads, cache->n_sessions), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3(cache->n_kv_heads, cache->n_sessions), dim3(64), 0, s, a);
  if ((st = launch_status("append"))) return st;
  hipLaunchKernelGGL(advance_kernel, dim3((cache->n_sessions + 255) / 256), dim3(256), 0, s,
                     const_cast<int32_t*>(cache->n_tokens), cache->n_sessions);
  return launch_status("advance");
}

int tq_retier_pages(const tq_layer* layer, const tq_cache* cache, const int64_t* page_index,
                    const uint64_t* new_desc, int n, int sources, int32_t* error_flags, void* stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "negative page count");
  if (sources & ~(TQ_RETIER_FROM_PACKED | TQ_RETIER_FROM_FP16))
    return fail(TQ_ERR_INVALID_ARG, "unknown source bits %#x", sources);
  if (n == 0) return TQ_OK;
  if (!page_index || !new_desc) return fail(TQ_ERR_INVALID_ARG, "null page list");
  if (((uintptr_t)page_index & 7) || ((uintptr_t)new_desc & 7))
    return fail(TQ_ERR_ALIGNMENT, "page lists must be 8-byte aligned");
  if (((uintptr_t)error_flags & 3) != 0) return fail(TQ_ERR_ALIGNMENT, "error_flags misaligned");
  RetierArgs a;
  a.index = page_index;
  a.new_desc = new_desc;
  a.n = n;
  a.sources = sources == 0 ? (TQ_RETIER_FROM_PACKED | TQ_RETIER_FROM_FP16) : sources;
  a.err = error_flags;
  a.pages = const_cast<uint64_t*>(cache->pages);
  a.n_entries = (int64_t)cache->n_sessions * cache->n_kv_heads * cache->max_pages;
  a.pool = reinterpret_cast<char*>(cache->pool);
  a.pool_bytes = cache->pool_bytes;
  a.sign_mask = layer->sign_mask;
  a.k_table = layer->k_table;
  a.v_table = layer->v_table;
  a.qjl_s = layer->qjl_s;
  a.k_polar = layer->k_codebook == TQ_CODEBOOK_POLAR;
  a.v_polar = layer->v_codebook == TQ_CODEBOOK_POLAR;
  // packed sources first: the pages it re-tiers no longer look like fp16
  // pages to the second launch.  The first launch raises the error flags.
  const dim3 grid(std::min(n, kRetierBlocks));
  a.raise_errors = 1;
  if (a.sources & TQ_RETIER_FROM_PACKED) {
    hipLaunchKernelGGL((retier_kernel<false, false>), grid, dim3(64), 0, (hipStream_t)stream, a);
    if ((st = launch_status("retier packed pages"))) return st;
    a.raise_errors = 0;
  }
  if (a.sources & TQ_RETIER_FROM_FP16) {
    if (a.k_polar || a.v_polar)
      hipLaunchKernelGGL((retier_kernel<true, true>), grid, dim3(64), 0, (hipStream_t)stream, a);
    else
      hipLaunchKernelGGL((retier_kernel<true, false>), grid, dim3(64), 0, (hipStream_t)stream, a);
    st = launch_status("retier fp16 pages");
  }
  return st;
}

}  // extern "C"
