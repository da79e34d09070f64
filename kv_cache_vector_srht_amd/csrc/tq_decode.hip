// Decode-attention kernels of libtq for gfx950 (CDNA4, wave64) and
// tq_decode_attention.
//
// (1) query prep rotates each query head (R q, and S q for QJL), pre-scaled
// for exp2; (2) split-K: a 4-wave workgroup per (session, KV head, page
// range); per page, lane = token for the key scores of the G query heads of
// the KV head (codes looked up two at a time in LDS tables, query coordinates
// read as wave-uniform scalars), an online softmax with wavefront reductions,
// then lane = (token quarter, 8 coordinates) for the value accumulation in the
// rotated domain; (3) combine: log-sum-exp merge of the splits and one inverse
// rotation per query head (the Walsh-Hadamard transform factored out of the
// value sum, as the MLX TurboQuant skill page reports for its Metal kernels,
// Path A > Optimisations Metal).
#include <atomic>
#include <cstring>
#include <type_traits>

#include "tq_device.h"

namespace tq {
namespace dev {
namespace {

// ------------------------------------------------------------------ decode
struct DecodeArgs {
  const void* q;
  int q_dtype;
  int64_t q_sb, q_sh;
  int n_q_heads, group;
  float scale2;  // softmax scale * log2(e)
  int qjl_sign;  // TQ_QJL_SCORE_SIGN: the query side of the QJL term is sign(S q)
  int k_polar, v_polar;   // PolarQuant parts: pages wider than 4 bits are skipped
  const int32_t* n_tokens;
  int n_sessions, n_kv_heads, max_pages;
  const char* pool;
  uint64_t pool_bytes;
  const uint32_t* sign_mask;
  const float* k_table;
  const float* v_table;
  const float* qjl_s;
  int n_splits, pages_per_split;            // common class
  int n_splits_general, pages_per_split_general;   // other class
  int n_splits_wide, pages_per_split_wide;         // wide class
  int part_base[3], n_partials;                     // first partial of each class, total
  int other_edges_first;        // merged launch: the other class's middle ranges after the others
  float* wsq;   // [B][H_q][384]: rotated q, plain q, S q (pre-scaled)
  float* wsp;   // [B][H_q][n_splits][kPartialFloats]: m, l, -, -, acc[128]
  float* out;
  float* mass;  // [B][H_q][max_pages] page attention mass, or null
  float* tmass; // [B][H_q][max_pages * 64] token attention weights, or null (then mass is null)
  // bit u of unit_skip[c]: class c was not launched for unit u = b * H_kv + h
  // (its partials of that class hold nothing; the combine passes over them)
  uint32_t unit_skip[3][TQ_MAX_LISTED_UNITS / 32];
};

// The units (b * H_kv + h) one split launch covers.  A single-class launch
// takes one unit per grid row.  The merged launch (CLASS 3) runs up to three
// groups of units: group[2] units of the other class, then group[1] of the
// wide class, then group[0] of the common class, listed in that order in
// unit[] (a class absent from the launch has an empty group).  n == 0: no
// list, unit index = position in the group (single-class: the grid's rows).
struct UnitList {
  int32_t n;
  int32_t group[3];
  uint16_t unit[2 * TQ_MAX_LISTED_UNITS];
};

// In-place Walsh-Hadamard transform (Sylvester order, unnormalised) of 128
// values held one per thread by the block's first two waves (thread j holds
// value j, active = j < 128): stages 1..32 inside the wave through lane
// shuffles, stage 64 across the two waves through `xch` (128 floats of LDS).
// Every thread of the block calls it: it holds one barrier.
__device__ __forceinline__ float fwht128_two_waves(float v, int j, bool active, float* xch) {
  if (active) {
#pragma clang loop unroll(full)
    for (int hh = 1; hh < 64; hh <<= 1) {
      const float other = __shfl_xor(v, hh, 64);
      v = (j & hh) ? other - v : v + other;
    }
    xch[j] = v;
  }
  __syncthreads();
  if (active) {
    const float other = xch[j ^ 64];
    v = (j & 64) ? other - v : v + other;
  }
  return v;
}

// (1) query prep: one 128-thread block per (session, query head).
__global__ __launch_bounds__(128) void qprep_kernel(DecodeArgs a) {
  __shared__ float buf[D];
  __shared__ float qs[D];
  const int j = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / a.n_q_heads, h = row - b * a.n_q_heads;
  const float qj = load_elem(a.q, a.q_dtype, (size_t)b * a.q_sb + (size_t)h * a.q_sh + j);
  if (a.mass) {
    // pages no split kernel visits keep -inf (mass 0 after the combine)
    float* mrow = a.mass + (size_t)row * a.max_pages;
    for (int p = j; p < a.max_pages; p += 128) mrow[p] = -INFINITY;
  }
  if (a.tmass) {
    // so do the tokens of such pages
    float4* trow = reinterpret_cast<float4*>(a.tmass + (size_t)row * a.max_pages * PT);
    for (int i = j; i < a.max_pages * PT / 4; i += 128) trow[i] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  }
  const uint32_t neg = (a.sign_mask[j >> 5] >> (j & 31)) & 1u;
  qs[j] = qj;
  const float hq = fwht128_two_waves(flip_if(qj, neg), j, true, buf);   // H D q
  // Layout per (session, KV head): three sections of 128 x G floats (rotated q,
  // plain q, S q), each ordered [coordinate / 4][query head in group][coordinate % 4]
  // so that one 16-dword scalar load brings 4 coordinates of 4 heads.
  const int G = a.group, g = h / G, hg = h - g * G;
  float* w = a.wsq + ((size_t)b * a.n_kv_heads + g) * kQPrepFloats * G;
  const size_t slot = ((size_t)(j >> 2) * G + hg) * 4 + (j & 3);
  // R q = D H D q / sqrt(d); packed-page scores use (R q) * scale2 / sqrt(d).
  w[slot] = flip_if(hq, neg) * (a.scale2 * (1.0f / D));
  w[D * G + slot] = qj * a.scale2;
  if (a.qjl_s) {
    const float* srow = a.qjl_s + (size_t)j * D;
    float p = 0.f;
    for (int i = 0; i < D; ++i) p = fmaf(srow[i], qs[i], p);
    if (a.qjl_sign) {
      // sign agreement scaled by pi/2 ||q|| / m (every thread sums the same
      // squares in the same order)
      float qq = 0.f;
#pragma clang loop unroll(disable)
      for (int i = 0; i < D; ++i) qq = fmaf(qs[i], qs[i], qq);
      w[2 * D * G + slot] = (p >= 0.f ? 1.f : -1.f) * sqrtf(qq) * (a.scale2 * kHalfPi / TQ_JL_DIM);
    } else {
      w[2 * D * G + slot] = p * (a.scale2 * kSqrtHalfPi / TQ_JL_DIM);
    }
  } else {
    w[2 * D * G + slot] = 0.f;
  }
}

// Row stride (floats) of a wave's page weights in LDS, [head][token]: four
// floats past a page, so that the four head rows a matrix-core step reads
// at once (lane % 4 picks the row) fall in different LDS banks.
constexpr int kWRow = PT + 4;

// The query's key table for 1- and 2-bit keys of the common class (up to 4
// query heads): a stream nibble covers four 1-bit or two 2-bit codes, and
// entry 16 g + m holds, per head, the score of nibble value m at nibble
// position g (coordinates 4g .. 4g + 3, resp. 2g, 2g + 1).
constexpr int kKeyLutEntries = 64 * 16;

// Per-workgroup LDS of the split kernel (KLUT: the launch may build the key
// table; the others leave its space out).
template <bool KLUT>
struct SplitTables {
  float2 kpair[340];          // pair tables for bits 1..4 (4 + 16 + 64 + 256 entries)
  float2 vpair[340];
  union {
    float4 kquad[272];        // quad tables for bits 1..2 (16 + 256 entries)
    float4 klut[KLUT ? kKeyLutEntries : 1];   // or the query's key table of 1- or 2-bit pages
  };
  float4 vquad[272];
  union {
    struct {
      float kcent[512];       // centroid lists for every bit width (table layout; 5-8 bits)
      float vcent[512];
    };
    uint4 kqa[256];           // or (common class, 1-4 bits) the query as the matrix
                              // cores' A operand (key_scores_mfma)
  };
};
template <int G, bool KLUT>
struct SplitLds {
  // the codebook tables serve the page loop; the workgroup reduction reuses
  // their space once every wave has left the loop (after a barrier)
  union {
    SplitTables<KLUT> t;
    float red[kDecodeWaves][G * D];
  };
  float w[kDecodeWaves][(G < 4 ? 4 : G) * kWRow];   // weights of the current page, [head][token]
                                                 // (rows G..3 stay zero)
  float stat[kDecodeWaves][2][G];          // m, l per wave
  int widths[kDecodeWaves];                // page widths each wave's descriptors hold
  uint64_t desc[kMaxPagesPerSplit];        // the range's page descriptors, read once
};

__device__ __forceinline__ int pair_offset(int b) {
  return b == 1 ? 0 : b == 2 ? 4 : b == 3 ? 20 : 84;
}

// Up to 2 bits, four consecutive codes (4B bits, the first in the low bits)
// index one table entry holding their four centroids.
__device__ __forceinline__ int quad_offset(int b) { return b == 1 ? 0 : 16; }

// Key scores of one packed page, lane = token: s[h] = sum_j qr[h][j] c[code_j].
// Query values are wave-uniform scalar loads; they share the LGKM counter with
// the LDS codebook lookups and return out of order, so the loop is pipelined by
// hand: for chunk n the first FMA waits for chunk n's data only, then chunk
// n+1's scalar loads and lookups are issued, then the rest of chunk n runs.
// The stream's words come in `sw` (its first 4B dwords are used).
template <int B, int G, int N>
__device__ __forceinline__ void key_scores_w(const uint32_t (&sw)[N], const float* __restrict__ qr,
                                             const float2* pair, const float4* quad, const float* cent,
                                             float (&s)[G]) {
  static_assert(N >= 4 * B, "the stream's words");
  constexpr int CH = G >= 8 ? 4 : 8;          // coordinates per chunk (its query values
                                              // take 2 x G x CH scalar registers)
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) s[h] = 0.f;
  float qa[G][CH], qb[G][CH], ca[CH], cb[CH];
  auto fetch = [&](int n, float (&qd)[G][CH], float (&cd)[CH]) {
    // prepared query: groups of four coordinates, all heads of a group together
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h)
#pragma clang loop unroll(full)
      for (int e = 0; e < CH; ++e) qd[h][e] = qr[((n * CH / 4 + (e >> 2)) * G + h) * 4 + (e & 3)];
    if constexpr (B <= 2) {
#pragma clang loop unroll(full)
      for (int e = 0; e < CH; e += 4) {
        const float4 c = quad[quad_offset(B) + checked(bits_at(sw, (n * CH + e) * B, 4 * B), 1 << (4 * B), kCheckDecodeTable)];
        cd[e] = c.x;
        cd[e + 1] = c.y;
        cd[e + 2] = c.z;
        cd[e + 3] = c.w;
      }
    } else if constexpr (B <= 4) {
      const float2* pt = pair + pair_offset(B);
#pragma clang loop unroll(full)
      for (int e = 0; e < CH; e += 2) {
        const float2 c = pt[checked(bits_at(sw, (n * CH + e) * B, 2 * B), 1 << (2 * B), kCheckDecodeTable)];
        cd[e] = c.x;
        cd[e + 1] = c.y;
      }
    } else {
      const float* ct = cent + centroid_offset(B);
#pragma clang loop unroll(full)
      for (int e = 0; e < CH; ++e) cd[e] = ct[checked(bits_at(sw, (n * CH + e) * B, B), 1 << B, kCheckDecodeTable)];
    }
  };
  auto fmas = [&](const float (&qd)[G][CH], const float (&cd)[CH], int e0, int e1) {
#pragma clang loop unroll(full)
    for (int e = e0; e < e1; ++e)
#pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) s[h] = fmaf(qd[h][e], cd[e], s[h]);
  };
  fetch(0, qa, ca);
#pragma clang loop unroll(full)
  for (int n = 0; n < D / CH; n += 2) {
    fmas(qa, ca, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    fetch(n + 1, qb, cb);
    __builtin_amdgcn_sched_barrier(0);
    fmas(qa, ca, 1, CH);
    fmas(qb, cb, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (n + 2 < D / CH) fetch(n + 2, qa, ca);
    __builtin_amdgcn_sched_barrier(0);
    fmas(qb, cb, 1, CH);
  }
}

template <int B, int G>
__device__ __forceinline__ void key_scores(const char* blk, int lane, const float* __restrict__ qr,
                                           const float2* pair, const float4* quad, const float* cent,
                                           float (&s)[G]) {
  uint32_t sw[4 * B];
  const uint4* src = reinterpret_cast<const uint4*>(blk);
#pragma clang loop unroll(full)
  for (int w = 0; w < B; ++w) {
    const uint4 v = src[w * 64 + lane];
    sw[4 * w] = v.x; sw[4 * w + 1] = v.y; sw[4 * w + 2] = v.z; sw[4 * w + 3] = v.w;
  }
  key_scores_w<B, G>(sw, qr, pair, quad, cent, s);
}

// Key scores of a 1- or 2-bit packed page from the query's key table, lane =
// token: s[h] = sum over the stream's nibbles g of klut[16 g + nibble].h (one
// lookup of four heads and G additions per nibble, against 4 (B = 1) or 2
// (B = 2) coordinates' decode and G multiply-adds each).
template <int B, int G, int N>
__device__ __forceinline__ void key_scores_table(const uint32_t (&sw)[N], const float4* klut, float (&s)[G]) {
  static_assert(B == 1 || B == 2, "a nibble holds whole codes");
  static_assert(N >= 4 * B, "the stream's words");
  constexpr int kGroups = 32 * B;
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma clang loop unroll(full)
  for (int g = 0; g < kGroups; ++g) {
    const float4 v = klut[checked(16 * g + (int)((sw[g >> 3] >> (4 * (g & 7))) & 0xFu), kKeyLutEntries, kCheckDecodeTable)];
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h) s[h] += vv[h];
  }
}

// Key scores of an fp16 page, lane = token, with the unrotated query.
template <int G>
__device__ __forceinline__ void key_scores_fp16(const char* page, int lane, const float* __restrict__ qo,
                                                float (&s)[G]) {
  const __half* krow = reinterpret_cast<const __half*>(page) + (size_t)lane * D;
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma clang loop unroll(full)
  for (int c = 0; c < D / 8; ++c) {
    const uint4 kv = reinterpret_cast<const uint4*>(krow)[c];
    const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma clang loop unroll(full)
    for (int e = 0; e < 4; ++e) {
      const float2 f = __half22float2(*reinterpret_cast<const __half2*>(&kw[e]));
      const int j = 8 * c + 2 * e;
#pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) {
        s[h] = fmaf(qo[((j >> 2) * G + h) * 4 + (j & 3)], f.x, s[h]);
        s[h] = fmaf(qo[((j >> 2) * G + h) * 4 + (j & 3) + 1], f.y, s[h]);
      }
    }
  }
}

// QJL term: sum_i qs[h][i] (2 z_i - 1) for lane = token, taken as
// 2 sum_i z_i qs[h][i] - qsum[h] with z_i in {0, 1} (qsum[h] = sum_i qs[h][i]).
// Four consecutive sign bits x are spread into the four bytes of a register by
// one multiply, x * (1 + 2^7 + 2^14 + 2^21): bit b of x lands at b + 7m for the
// m-th term, positions that are all distinct (no carries), and only m = b hits
// bit 8b; each byte is then converted to float on its own.  That is 1.75
// instructions per coordinate for the signs, not the 3 of a per-bit select.
template <int G>
__device__ __forceinline__ void qjl_scores(const char* qb, int lane, const float* __restrict__ qsv,
                                           const float (&qsum)[G], float (&t)[G]) {
  const uint4 z4 = reinterpret_cast<const uint4*>(qb)[lane];
  const uint32_t zw[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) t[h] = 0.f;
#pragma clang loop unroll(full)
  for (int n = 0; n < TQ_JL_DIM / 4; ++n) {
    uint32_t by = ((zw[n >> 3] >> (4 * (n & 7))) & 0xFu) * 0x204081u & 0x01010101u;
    // opaque to the optimiser, which would otherwise extract every bit on its
    // own before converting it
    asm("" : "+v"(by));
#pragma clang loop unroll(full)
    for (int e = 0; e < 4; ++e) {
      const float z = (float)((by >> (8 * e)) & 0xFFu);   // sign bit 4 n + e
#pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) t[h] = fmaf(qsv[(n * G + h) * 4 + e], z, t[h]);
    }
  }
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) t[h] = fmaf(2.f, t[h], -qsum[h]);
}

// The same term from a table of signed sums per group of four sign bits:
// lut[(n * 16 + v) * G + h] = sum_{e < 4} (2 bit_e(v) - 1) qs[h][4 n + e], so a
// key's term is 32 reads (all G heads of one group at once) and their sums.
template <int G>
__device__ __forceinline__ void qjl_scores_lut(const char* qb, int lane, const float* lut, float (&t)[G]) {
  const uint4 z4 = reinterpret_cast<const uint4*>(qb)[lane];
  const uint32_t zw[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) t[h] = 0.f;
#pragma clang loop unroll(full)
  for (int n = 0; n < TQ_JL_DIM / 4; ++n) {
    const uint32_t v = (zw[n >> 3] >> (4 * (n & 7))) & 0xFu;
    const float* e = lut + (n * 16 + (int)v) * G;
    if constexpr (G % 4 == 0) {
#pragma clang loop unroll(full)
      for (int h = 0; h < G; h += 4) {
        const float4 x = *reinterpret_cast<const float4*>(e + h);
        t[h] += x.x;
        t[h + 1] += x.y;
        t[h + 2] += x.z;
        t[h + 3] += x.w;
      }
    } else if constexpr (G == 2) {
      const float2 x = *reinterpret_cast<const float2*>(e);
      t[0] += x.x;
      t[1] += x.y;
    } else {
      t[0] += e[0];
    }
  }
}

typedef float v4f __attribute__((ext_vector_type(4)));

// Value sums of one packed page on the matrix cores (v_mfma_f32_4x4x1f32, 16
// independent 4 x 4 outer products per instruction, exact float32 products).
// Per token t: lane L (block L / 4, column L % 4) brings the value of its V
// stream's first coordinate (then its second) as the B operand, and the A
// operand p'[4 g + L % 4][t], the weight (times the token's norm) of query head
// 4 g + L % 4, from the wave's weight rows in LDS (rows past the group are
// zero); register i of acc[g][k] of lane L then accumulates head 4 g + i,
// coordinate v_stream_coord(L, k).  Codes of stream L: positions 2t, 2t + 1.
template <int B, int NG, int N>
__device__ __forceinline__ void value_mfma_w(const uint32_t (&sw)[N], int lane, const float* wv,
                                             const float2* pair, const float4* quad,
                                             v4f (&acc)[NG][2]) {
  static_assert(N >= 4 * B, "the stream's words");
  const float* wl = wv + (lane & 3) * kWRow;
  // four tokens per step; step u + 1's weights and centroids are read from LDS
  // while step u's products run (LDS reads complete in order, so the wait
  // before step u's products leaves step u + 1's reads in flight)
  float4 wa[NG], wb[NG];
  float ca[8], cb[8];   // per token pair: (t, first), (t, second), (t + 1, first), (t + 1, second)
  auto fetch = [&](int t4, float4 (&wd)[NG], float (&cd)[8]) {
#pragma clang loop unroll(full)
    for (int g = 0; g < NG; ++g) wd[g] = *reinterpret_cast<const float4*>(wl + 4 * g * kWRow + 4 * t4);
#pragma clang loop unroll(full)
    for (int e = 0; e < 4; e += 2) {
      const int t = 4 * t4 + e;
      if constexpr (B <= 2) {
        const float4 q = quad[quad_offset(B) + checked(bits_at(sw, 2 * t * B, 4 * B), 1 << (4 * B), kCheckDecodeTable)];
        cd[2 * e] = q.x; cd[2 * e + 1] = q.y; cd[2 * e + 2] = q.z; cd[2 * e + 3] = q.w;
      } else {
        const float2* pt = pair + pair_offset(B);
        const float2 p0 = pt[checked(bits_at(sw, 2 * t * B, 2 * B), 1 << (2 * B), kCheckDecodeTable)];
        const float2 p1 = pt[checked(bits_at(sw, 2 * (t + 1) * B, 2 * B), 1 << (2 * B), kCheckDecodeTable)];
        cd[2 * e] = p0.x; cd[2 * e + 1] = p0.y; cd[2 * e + 2] = p1.x; cd[2 * e + 3] = p1.y;
      }
    }
  };
  auto products = [&](const float4 (&wd)[NG], const float (&cd)[8]) {
#pragma clang loop unroll(full)
    for (int e = 0; e < 4; e += 2)
#pragma clang loop unroll(full)
      for (int g = 0; g < NG; ++g) {
        const float a0 = e == 0 ? wd[g].x : wd[g].z, a1 = e == 0 ? wd[g].y : wd[g].w;
        acc[g][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(a0, cd[2 * e], acc[g][0], 0, 0, 0);
        acc[g][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a0, cd[2 * e + 1], acc[g][1], 0, 0, 0);
        acc[g][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(a1, cd[2 * e + 2], acc[g][0], 0, 0, 0);
        acc[g][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a1, cd[2 * e + 3], acc[g][1], 0, 0, 0);
      }
  };
  fetch(0, wa, ca);
#pragma clang loop unroll(full)
  for (int t4 = 0; t4 < PT / 4; t4 += 2) {
    __builtin_amdgcn_sched_barrier(0);
    fetch(t4 + 1, wb, cb);
    __builtin_amdgcn_sched_barrier(0);
    products(wa, ca);
    __builtin_amdgcn_sched_barrier(0);
    if (t4 + 2 < PT / 4) fetch(t4 + 2, wa, ca);
    __builtin_amdgcn_sched_barrier(0);
    products(wb, cb);
  }
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }

// Two float32 values as float16 parts: hi = fp16(y), lo = fp16(y - hi), the
// pair's hi parts in one dword (first value in the low half), lo in another.
// (fp16(y - hi) is y - hi rounded once: y - hi is exact in float32.)
__device__ __forceinline__ uint2 split_half2(float y0, float y1) {
  const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
  const _Float16 l0 = (_Float16)(y0 - (float)h0), l1 = (_Float16)(y1 - (float)h1);
  return make_uint2((uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16),
                    (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16));
}

// Scale of the key pair table on the matrix cores: coordinates of a unit
// vector times sqrt(d) stay below 12 in magnitude, so 2^8 keeps them well
// inside the float16 range while their lo parts stay normal.
constexpr float kKeyPairScale = 256.f;


// Code words of a 3- or 4-bit key page in the layout key_scores_mfma reads:
// lane l (k-group g = l / 16, column n = l % 16) takes the coordinate quarter
// 32 g .. 32 g + 31 of token 16 t + n for each tile t, i.e. dwords B g ..
// B g + B - 1 of that token's stream, into kw[B t ..].
template <int B>
__device__ __forceinline__ void load_keys_mfma(const char* kp, int lane, uint32_t (&kw)[16]) {
  const int g = lane >> 4, n = lane & 15;
  if constexpr (B == 4) {
    const uint4* ks = reinterpret_cast<const uint4*>(kp);
#pragma clang loop unroll(full)
    for (int t = 0; t < 4; ++t) {
      const uint4 x = ks[g * 64 + 16 * t + n];
      kw[4 * t] = x.x; kw[4 * t + 1] = x.y; kw[4 * t + 2] = x.z; kw[4 * t + 3] = x.w;
    }
  } else {
    // a quarter is 96 bits: dwords 3 g .. 3 g + 2, which may straddle the
    // stream's 16-byte blocks (dword d of token u: block d / 4, lane u)
    const uint32_t* kd = reinterpret_cast<const uint32_t*>(kp);
#pragma clang loop unroll(full)
    for (int t = 0; t < 4; ++t)
#pragma clang loop unroll(full)
      for (int i = 0; i < 3; ++i) {
        const int d = 3 * g + i;
        kw[3 * t + i] = kd[((d >> 2) * 64 + 16 * t + n) * 4 + (d & 3)];
      }
#pragma clang loop unroll(full)
    for (int i = 12; i < 16; ++i) kw[i] = 0;
  }
}

// Key scores of a 3- or 4-bit packed page for four query heads on the matrix
// cores (v_mfma_f32_16x16x32_f16), lane = token on return, unscaled (times
// the query's and the table's scales).  The page is four tiles of 16 tokens:
// tile t is the B operand (column n = token 16 t + n) and the query the A
// operand (row i = head i % 4, each head four times), so accumulator t holds
// in lane l the scores of token 16 t + l % 16 for the four heads, and lane l
// keeps accumulator l / 16, its own token's.  Float32 operands enter as
// float16 hi and lo parts and each product as three float16 ones (hi hi,
// hi lo, lo hi), exact in the float32 accumulator; the dropped lo lo term and
// the lo parts' rounding are below 2^-21 of each product.  In step st (of 8)
// k-group g = l / 16 holds coordinates c0..c3 = 32 g + 4 st + 0..3, two code
// pairs, as B = [ch0 ch1 cl0 cl1 ch2 ch3 cl2 cl3]: each pair's (hi, lo) table
// entry (khl, two dwords) is one lookup into its place.  The query is
// A1 = [qh0 qh1 qh0 qh1 qh2 qh3 qh2 qh3] (qh ch + qh cl) and
// A2 = [ql0 ql1 0 0 ql2 ql3 0 0] (ql ch), staged in kqa per (st, g, head).
template <int B>
__device__ __forceinline__ void key_scores_mfma(const uint32_t (&kw)[16], int lane, const uint4* kqa,
                                                const uint2* khl, float (&s)[4]) {
  static_assert(B == 3 || B == 4, "pair-table widths");
  const int g = lane >> 4;
  v4f acc[4];
#pragma clang loop unroll(full)
  for (int t = 0; t < 4; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma clang loop unroll(full)
  for (int st = 0; st < 8; ++st) {
    const uint4* qa = kqa + checked(2 * ((st * 4 + g) * 4 + (lane & 3)), 255, kCheckDecodeTable);
    const half8 a1 = as_half8(qa[0]), a2 = as_half8(qa[1]);
#pragma clang loop unroll(full)
    for (int t = 0; t < 4; ++t) {
      // the step's two code pairs (2 x 2B bits) of tile t's token: pairs
      // 2 st, 2 st + 1 of the lane's quarter (pair m at bit 2 B m)
      uint32_t x;
      if constexpr (B == 4) {
        x = kw[4 * t + (st >> 1)] >> (16 * (st & 1));
      } else {
        const int bit = 12 * st, d = bit >> 5, sh = bit & 31;
        x = sh <= 20 ? kw[3 * t + d] >> sh : __builtin_amdgcn_alignbit(kw[3 * t + d + 1], kw[3 * t + d], sh);
      }
      constexpr uint32_t kMask = (1u << (2 * B)) - 1u;
      const uint2 e0 = khl[checked((int)(x & kMask), 1 << (2 * B), kCheckDecodeTable)];
      const uint2 e1 = khl[checked((int)((x >> (2 * B)) & kMask), 1 << (2 * B), kCheckDecodeTable)];
      const half8 bv = as_half8(make_uint4(e0.x, e0.y, e1.x, e1.y));
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, bv, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bv, acc[t], 0, 0, 0);
    }
  }
#pragma clang loop unroll(full)
  for (int h = 0; h < 4; ++h)
    s[h] = g == 0 ? acc[0][h] : g == 1 ? acc[1][h] : g == 2 ? acc[2][h] : acc[3][h];
}

// Key scores of a packed page at 5-8 bits.  These widths are rare (a few
// important heads), so the code is kept short instead of fully unrolled: four
// passes over 32 coordinates each, whose codes fill exactly B dwords of the
// lane's stream (dwords B n .. B n + B - 1).
template <int B, int G>
__device__ __forceinline__ void key_scores_wide(const char* blk, int lane, const float* __restrict__ qr,
                                                const float* cent, float (&s)[G]) {
  constexpr int CH = 4;                       // coordinates per chunk, pipelined as in key_scores
  const uint32_t* src = reinterpret_cast<const uint32_t*>(blk);
  const float* ct = cent + centroid_offset(B);
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) s[h] = 0.f;
  // pass n + 1's dwords are loaded while pass n computes (the last pass
  // reloads its own, harmlessly)
  uint32_t w[B], nx[B];
  auto load = [&](int n, uint32_t (&d)[B]) {
#pragma clang loop unroll(full)
    for (int i = 0; i < B; ++i) {
      const int dd = B * n + i;
      d[i] = src[((dd >> 2) * 64 + lane) * 4 + (dd & 3)];
    }
  };
  load(0, w);
#pragma clang loop unroll(disable)
  for (int n = 0; n < 4; ++n) {
    load(min(n + 1, 3), nx);
    const float* qn = qr + 32 * G * n;
    float qa[G][CH], qb[G][CH], ca[CH], cb[CH];
    auto fetch = [&](int c, float (&qd)[G][CH], float (&cd)[CH]) {
#pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h)
#pragma clang loop unroll(full)
        for (int e = 0; e < CH; ++e) qd[h][e] = qn[(c * G + h) * CH + e];
#pragma clang loop unroll(full)
      for (int e = 0; e < CH; ++e) cd[e] = ct[checked(bits_at(w, (c * CH + e) * B, B), 1 << B, kCheckDecodeTable)];
    };
    auto fmas = [&](const float (&qd)[G][CH], const float (&cd)[CH], int e0, int e1) {
#pragma clang loop unroll(full)
      for (int e = e0; e < e1; ++e)
#pragma clang loop unroll(full)
        for (int h = 0; h < G; ++h) s[h] = fmaf(qd[h][e], cd[e], s[h]);
    };
    fetch(0, qa, ca);
#pragma clang loop unroll(full)
    for (int c = 0; c < 32 / CH; c += 2) {
      fmas(qa, ca, 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      fetch(c + 1, qb, cb);
      __builtin_amdgcn_sched_barrier(0);
      fmas(qa, ca, 1, CH);
      fmas(qb, cb, 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      if (c + 2 < 32 / CH) fetch(c + 2, qa, ca);
      __builtin_amdgcn_sched_barrier(0);
      fmas(qb, cb, 1, CH);
    }
#pragma clang loop unroll(full)
    for (int i = 0; i < B; ++i) w[i] = nx[i];
  }
}

template <int B, int NG>
__device__ __forceinline__ void value_mfma(const char* blk, int lane, const float* wv,
                                           const float2* pair, const float4* quad,
                                           v4f (&acc)[NG][2]) {
  uint32_t sw[4 * B];
  const uint4* src = reinterpret_cast<const uint4*>(blk);
#pragma clang loop unroll(full)
  for (int w = 0; w < B; ++w) {
    const uint4 v = src[w * 64 + lane];
    sw[4 * w] = v.x; sw[4 * w + 1] = v.y; sw[4 * w + 2] = v.z; sw[4 * w + 3] = v.w;
  }
  value_mfma_w<B, NG>(sw, lane, wv, pair, quad, acc);
}

// Value sums of a packed page at 5-8 bits, as value_mfma with one centroid
// lookup per code, in four passes of 16 tokens: a pass's 32 codes of the
// stream are exactly B dwords (B n .. B n + B - 1), loaded one pass ahead.
template <int B, int NG>
__device__ __forceinline__ void value_mfma_wide(const char* blk, int lane, const float* wv, const float* cent,
                                                v4f (&acc)[NG][2]) {
  const uint32_t* src = reinterpret_cast<const uint32_t*>(blk);
  const float* ct = cent + centroid_offset(B);
  const float* wl = wv + (lane & 3) * kWRow;
  uint32_t w[B], nx[B];
  auto load = [&](int n, uint32_t (&d)[B]) {
#pragma clang loop unroll(full)
    for (int i = 0; i < B; ++i) {
      const int dd = B * n + i;
      d[i] = src[((dd >> 2) * 64 + lane) * 4 + (dd & 3)];
    }
  };
  load(0, w);
#pragma clang loop unroll(disable)
  for (int n = 0; n < 4; ++n) {
    load(min(n + 1, 3), nx);
#pragma clang loop unroll(full)
    for (int t4 = 0; t4 < 4; ++t4) {
      float4 a[NG];
#pragma clang loop unroll(full)
      for (int g = 0; g < NG; ++g) a[g] = *reinterpret_cast<const float4*>(wl + 4 * g * kWRow + 16 * n + 4 * t4);
#pragma clang loop unroll(full)
      for (int e = 0; e < 4; ++e) {
        const int tl = 4 * t4 + e;   // token 16 n + tl: codes at pass positions 2 tl, 2 tl + 1
        const float c0 = ct[checked(bits_at(w, 2 * tl * B, B), 1 << B, kCheckDecodeTable)];
        const float c1 = ct[checked(bits_at(w, (2 * tl + 1) * B, B), 1 << B, kCheckDecodeTable)];
#pragma clang loop unroll(full)
        for (int g = 0; g < NG; ++g) {
          const float av = e == 0 ? a[g].x : e == 1 ? a[g].y : e == 2 ? a[g].z : a[g].w;
          acc[g][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(av, c0, acc[g][0], 0, 0, 0);
          acc[g][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(av, c1, acc[g][1], 0, 0, 0);
        }
      }
    }
#pragma clang loop unroll(full)
    for (int i = 0; i < B; ++i) w[i] = nx[i];
  }
}

// Value sums of an fp16 page on the matrix cores, as value_mfma_w but in the
// original domain (the caller rotates the sums once, after the last page): the
// B operand of token t is its value at the lane's coordinates
// v_stream_coord(L, 0) and v_stream_coord(L, 0) + 1, one 4-byte load per token.
template <int NG>
__device__ __forceinline__ void value_mfma_fp16(const char* page, int lane, const float* wv,
                                                v4f (&acc)[NG][2]) {
  const __half2* vcol = reinterpret_cast<const __half2*>(page + PT * D * 2) + v_stream_coord(lane, 0) / 2;
  const float* wl = wv + (lane & 3) * kWRow;
#pragma clang loop unroll_count(4)
  for (int t4 = 0; t4 < PT / 4; ++t4) {
    float2 v[4];
#pragma clang loop unroll(full)
    for (int e = 0; e < 4; ++e) v[e] = __half22float2(vcol[(4 * t4 + e) * (D / 2)]);
#pragma clang loop unroll(full)
    for (int g = 0; g < NG; ++g) {
      const float4 wd = *reinterpret_cast<const float4*>(wl + 4 * g * kWRow + 4 * t4);
      const float w4[4] = {wd.x, wd.y, wd.z, wd.w};
#pragma clang loop unroll(full)
      for (int e = 0; e < 4; ++e) {
        acc[g][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(w4[e], v[e].x, acc[g][0], 0, 0, 0);
        acc[g][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(w4[e], v[e].y, acc[g][1], 0, 0, 0);
      }
    }
  }
}

// acc += D H D x for sums x held as the matrix-core value sums hold them (lane
// L: coordinates c = v_stream_coord(L, k), k = 0, 1): coordinate bit 0 is the
// register pair, and bits 1, 2, 3, 4, 5, 6 are lane bits 0, 1, 3, 4, 5, 2, so
// the unnormalised transform is one in-lane butterfly and six lane exchanges.
template <int NG>
__device__ __forceinline__ void add_rotated(const v4f (&x)[NG][2], int lane, const uint32_t* sign_mask,
                                            v4f (&acc)[NG][2]) {
  const int c0 = v_stream_coord(lane, 0);
  const uint32_t n0 = (sign_mask[c0 >> 5] >> (c0 & 31)) & 1u, n1 = (sign_mask[c0 >> 5] >> ((c0 + 1) & 31)) & 1u;
  constexpr int kLaneBit[6] = {0, 1, 3, 4, 5, 2};
#pragma clang loop unroll(full)
  for (int g = 0; g < NG; ++g)
#pragma clang loop unroll(full)
    for (int i = 0; i < 4; ++i) {
      const float y0 = flip_if(x[g][0][i], n0), y1 = flip_if(x[g][1][i], n1);
      float u0 = y0 + y1, u1 = y0 - y1;
#pragma clang loop unroll(full)
      for (int st = 0; st < 6; ++st) {
        const int m = 1 << kLaneBit[st];
        const float o0 = __shfl_xor(u0, m, 64), o1 = __shfl_xor(u1, m, 64);
        const float sg = (lane & m) ? -1.f : 1.f;
        u0 = fmaf(sg, u0, o0);
        u1 = fmaf(sg, u1, o1);
      }
      acc[g][0][i] += flip_if(u0, n0);
      acc[g][1][i] += flip_if(u1, n1);
    }
}

// Online-softmax update of one page for G heads.  s: log2-domain scores of
// this lane's token (-inf when masked); on return s holds p = 2^(s - m) and
// alpha the rescale of the running sums.  m is a wave-uniform reference, not
// necessarily the running maximum: it moves (to the exact maximum, with a
// rescale) only when a score exceeds it by more than kSoftmaxSlack, so most
// pages skip the 64-lane maximum reduction.  Every weight stays below
// 2^kSoftmaxSlack, far from float32 overflow even summed over 2^31 tokens;
// the partials carry their reference, and the log-sum-exp merges are exact
// for any reference, so only rounding differs from the running-maximum form.
constexpr float kSoftmaxSlack = 32.f;

template <int G>
__device__ __forceinline__ void softmax_update(float (&s)[G], float (&m)[G], float (&l)[G],
                                               float (&alpha)[G]) {
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) {
    // m = -inf (nothing seen yet): any unmasked lane moves it
    const bool up = __ballot(s[h] > m[h] + kSoftmaxSlack) != 0ull;
    const float mn = up ? fmaxf(m[h], wave_max(s[h])) : m[h];
    // the hardware exponential: a weight below 2^-126 of the reference (which
    // some token reached at weight 1) flushes to zero, far below any effect
    if (mn == -INFINITY) {
      alpha[h] = 1.f;
      s[h] = 0.f;
    } else {
      alpha[h] = up ? __builtin_amdgcn_exp2f(m[h] - mn) : 1.f;
      s[h] = __builtin_amdgcn_exp2f(s[h] - mn);
    }
    m[h] = mn;
    l[h] = fmaf(l[h], alpha[h], s[h]);
  }
}

// Page classes, each run by a kernel instantiation compiled for its formats
// alone (fewer code paths, fewer registers, more waves in flight):
//   0 common: k_bits, v_bits <= 4, no QJL;
//   1 wide:   k_bits, v_bits >= 5, no QJL (the few important heads);
//   2 other:  fp16 pages, QJL keys and mixed widths.
// Each writes its own partials; the combine merges them.  Beside common pages,
// the wide class (CLASS 3: common + wide) and also the other class (CLASS 4:
// all three) run in one merged launch, each block taking its class's copy of
// the page loop.  When a layer holds
// both common and wide pages, one launch (CLASS 3) runs the two classes' blocks
// side by side, so that the wide pages' latency hides behind common work.
__device__ __forceinline__ int page_class(int kb, int vb, bool qjl) {
  if (kb >= 1 && kb <= 4 && vb >= 1 && vb <= 4 && !qjl) return 0;
  if (kb >= 5 && vb >= 5 && !qjl) return 1;
  return 2;
}

// MASS: also write, per page and query head, log2 of the page's share of the
// softmax numerator (m + log2 of the page's sum of 2^(s - m)); the combine
// turns it into the page's attention mass.
template <int G, int CLASS, bool MASS>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(CLASS >= 3 || (CLASS == 0 && G <= 4) ? 4 : (CLASS == 2 && G <= 4) ? 3 : 1)))
void split_kernel(DecodeArgs a,
                                                                  const float* __restrict__ wsq,
                                                                  const uint64_t* __restrict__ pages,
                                                                  float* __restrict__ wsp,
                                                                  const UnitList list) {
  // the query's key table: common pages of up to four query heads
  constexpr bool kKeyTable = G <= 4 && (CLASS == 0 || CLASS >= 3);
  __shared__ SplitLds<G, kKeyTable> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the other class runs its ranges last page first: a decode loop's fp16
  // tail page is then in the first workgroups dispatched, not behind the
  // rounds of workgroups that find nothing of the class
  int split, hkv, b, cls = CLASS;
  if constexpr (CLASS >= 3) {
    // merged launch, one block per (unit, range): the other class's blocks
    // first, range-major from each unit's last range (where a decode loop's
    // fp16 tail page sits, so every unit's tail starts at once), then the wide
    // class's and the common class's blocks, unit-major.  With
    // other_edges_first only the other class's last and first ranges (the tail
    // and sink pages) come first, its middle ranges (empty around a decode
    // loop's tail) after the common blocks, range-major from the end.
    const int other_blocks = list.group[2] * a.n_splits_general;
    const int n_head = a.other_edges_first ? min(a.n_splits_general, 2) : a.n_splits_general;
    const int head_blocks = list.group[2] * n_head;
    const int wide_blocks = list.group[1] * a.n_splits_wide;
    const int common_blocks = (int)gridDim.x - other_blocks - wide_blocks;
    int i = blockIdx.x, pos, off;   // position in the class's group, its list offset
    if (i < head_blocks) {
      cls = 2;
      const int r = i / list.group[2];
      pos = i - r * list.group[2];
      split = a.other_edges_first && r == 1 ? 0 : a.n_splits_general - 1 - r;
      off = 0;
    } else if (i < head_blocks + wide_blocks) {
      cls = 1;
      i -= head_blocks;
      pos = i / a.n_splits_wide;
      split = i - pos * a.n_splits_wide;
      off = list.group[2];
    } else if (i < head_blocks + wide_blocks + common_blocks) {
      cls = 0;
      i -= head_blocks + wide_blocks;
      pos = i / a.n_splits;
      split = i - pos * a.n_splits;
      off = list.group[2] + list.group[1];
    } else {
      cls = 2;
      i -= head_blocks + wide_blocks + common_blocks;
      const int r = i / list.group[2];
      pos = i - r * list.group[2];
      split = a.n_splits_general - 2 - r;
      off = 0;
    }
    // without a list every group is every unit, in (B, H_kv) order
    const int u = list.n > 0 ? list.unit[off + pos] : pos;
    b = u / a.n_kv_heads;
    hkv = u - b * a.n_kv_heads;
  } else {
    split = CLASS == 2 ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
    hkv = blockIdx.y;
    b = blockIdx.z;
    if (list.n > 0) {
      const int u = list.unit[blockIdx.y];
      b = u / a.n_kv_heads;
      hkv = u - b * a.n_kv_heads;
    }
  }
  const int hq0 = hkv * G;
  // partials [B][H_q][n_partials]: the classes that run, in class order
  const size_t head_stride = (size_t)a.n_partials * kPartialFloats;
  float* part = wsp + ((size_t)b * a.n_q_heads + hq0) * head_stride +
                (size_t)checked(a.part_base[cls] + split, a.n_partials, kCheckDecodeIndex) * kPartialFloats;
  const int pps = cls == 0 ? a.pages_per_split : cls == 1 ? a.pages_per_split_wide : a.pages_per_split_general;

  const int ntok = max(0, a.n_tokens[b]);
  const int npages = min(a.max_pages, (ntok + PT - 1) / PT);   // never past the table row
  const int p_begin = split * pps;
  const int p_end = min(npages, p_begin + pps);
  const uint64_t* ptab = pages + ((size_t)b * a.n_kv_heads + hkv) * a.max_pages;
  const float* __restrict__ qrow = wsq + ((size_t)b * a.n_kv_heads + hkv) * kQPrepFloats * G;
  // A common-class range of four query heads with 3- or 4-bit keys scores them
  // on the matrix cores (key_scores_mfma): its key pair tables at those widths
  // hold float16 hi and lo parts (times kKeyPairScale), and the query is staged
  // as the A operand, times 2^E so that its largest magnitude is in [2^9, 2^10);
  // the scores are then multiplied by key_unscale = 2^-(E + 8).
  // (Not in the launch merged with the other class: its register budget is
  // spent by the other class's copy of the page loop.)
  constexpr bool kMfmaKeys = G == 4 && CLASS != 4;
  bool key_mfma = false;
  float key_unscale = 1.f;
  // A common-class block of four query heads stages the query as the matrix
  // cores' A operand before anything else (its loads then overlap the
  // descriptor scan's), whether or not its range holds 3- or 4-bit keys
  // (key_mfma, decided with the tables, says whether they are used).
  if constexpr (kMfmaKeys) {
    if (cls == 0) {
      // every wave finds the same largest magnitude of the prepared query
      float mx = 0.f;
      for (int i = lane; i < D * G; i += 64) mx = fmaxf(mx, fabsf(qrow[i]));
      mx = wave_max(mx);
      int ex = 0;
      (void)frexpf(mx, &ex);
      const int E = (mx > 0.f && mx <= 3.0e38f) ? min(60, max(-60, 10 - ex)) : 0;
      const float qs = ldexpf(1.f, E);
      key_unscale = ldexpf(1.f, -(E + 8));
      // entry (step st, k-group g, head h): coordinates c0..c3 = 32 g + 4 st
      // + 0..3 of head h as A1 = (qh0 qh1, qh0 qh1, qh2 qh3, qh2 qh3) and
      // A2 = (ql0 ql1, 0, ql2 ql3, 0), key_scores_mfma's operands (the
      // prepared query's layout: coordinate j of head h at ((j / 4) G + h)
      // 4 + j % 4, so c0..c3 are one aligned quad)
      if (tid < 128) {
        const int st = tid >> 4, gg = (tid >> 2) & 3, h = tid & 3;
        const int j0 = 32 * gg + 4 * st;
        const float* qc = qrow + ((j0 >> 2) * G + h) * 4;
        const uint2 v01 = split_half2(qc[0] * qs, qc[1] * qs);
        const uint2 v23 = split_half2(qc[2] * qs, qc[3] * qs);
        sm.t.kqa[checked(2 * tid, 256, kCheckDecodeTable)] = make_uint4(v01.x, v01.x, v23.x, v23.x);
        sm.t.kqa[checked(2 * tid + 1, 256, kCheckDecodeTable)] = make_uint4(v01.y, 0u, v23.y, 0u);
      }
    }
  }
  // A common-class block also loads the 1-4-bit pair and quad sources of both
  // tables before the descriptor scan (one pair of the 4-bit table per
  // thread, the 3-bit table in the first 64, a 2-bit quad's two pairs, a
  // 1-bit quad's in the first 16); the staging below writes those its widths
  // use.
  static_assert(64 * kDecodeWaves == 256, "one 4-bit pair per thread");
  struct PairSrc {
    float2 p3, p4, q2a, q2b, q1a, q1b;
  };
  PairSrc pre[2];
  const bool prefetched = (CLASS == 0 || CLASS >= 3) && cls == 0;
  if (prefetched) {
#pragma clang loop unroll(full)
    for (int kv = 0; kv < 2; ++kv) {
      const float2* pt = reinterpret_cast<const float2*>((kv ? a.v_table : a.k_table) + kPairOffset);
      pre[kv].p4 = pt[pair_offset(4) + tid];
      pre[kv].p3 = pt[pair_offset(3) + (tid & 63)];
      pre[kv].q2a = pt[pair_offset(2) + (tid & 15)];
      pre[kv].q2b = pt[pair_offset(2) + (tid >> 4)];
      pre[kv].q1a = pt[pair_offset(1) + (tid & 3)];
      pre[kv].q1b = pt[pair_offset(1) + ((tid >> 2) & 3)];
    }
  }
  bool need_tables;
  {
    // nothing of this class in the range: an empty partial, no setup (the
    // descriptors are read in parallel, one per thread)
    bool mine = false, coded = false;
    int widths = 0;   // bit b: a packed page of the class with K width b; bit 9 + b: V width b
    for (int p = p_begin + tid; p < p_end; p += blockDim.x) {
      const uint64_t raw = ptab[p];
      sm.desc[checked(p - p_begin, kMaxPagesPerSplit, kCheckDecodeIndex)] = raw;   // the page loop reads it from LDS
      const PageDesc pd = read_desc(raw);
      const bool m = page_class(pd.kb, pd.vb, pd.qjl) == cls;
      mine |= m;
      coded |= m && pd.kb != 0;
      if (m && pd.kb != 0 && pd.kb <= 8 && pd.vb <= 8) widths |= (1 << pd.kb) | (1 << (9 + pd.vb));
    }
#pragma clang loop unroll(full)
    for (int o = 1; o < 64; o <<= 1) widths |= __shfl_xor(widths, o, 64);
    __syncthreads();   // the cached descriptors are visible to every wave
    if (lane == 0) sm.widths[wave] = widths;
    need_tables = cls != 2 || __syncthreads_or(coded);
    if (!__syncthreads_or(mine)) {   // (also makes sm.widths visible)
      if (tid < G) {
        part[tid * head_stride] = -INFINITY;
        part[tid * head_stride + 1] = 0.f;
      }
      return;
    }
  }


  // Stage the codebook tables the range's pages of this class use: pair
  // tables at 3-4 bits, quad tables at 1-2 bits, centroid lists at 5-8 bits
  // (nothing when those pages are all fp16, as a decode loop's tail pages are).
  // A common-class range whose keys are 1 or 2 bits wide (one of the two, up
  // to 4 query heads, scalar codebooks) builds the query's key table for that
  // width instead of the key quad table (key_table_bits).
  int key_table_bits = 0;
  auto stage_tables = [&]() {
    if (!need_tables) return;
    int widths = 0;
#pragma clang loop unroll(full)
    for (int w = 0; w < kDecodeWaves; ++w) widths |= sm.widths[w];
    if (kKeyTable && cls == 0 && !a.k_polar) {
      const int k12 = widths & 6;
      key_table_bits = k12 == 2 ? 1 : k12 == 4 ? 2 : 0;
    }
    if constexpr (kMfmaKeys) {
      key_mfma = cls == 0 && (widths & 0x18) != 0;
    }
    if (kKeyTable && key_table_bits) {
      // entry 16 g + m: sum over the nibble's codes of q[h][coordinate] c[code],
      // the prepared query (scale included) at qrow[((j / 4) G + h) 4 + j % 4]
      const float* cb = a.k_table + centroid_offset(key_table_bits);
      const int n = 16 * 32 * key_table_bits;
      for (int i = tid; i < n; i += blockDim.x) {
        const int g = i >> 4, mm = i & 15;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma clang loop unroll(full)
        for (int h = 0; h < G; ++h) {
          if (key_table_bits == 1) {
#pragma clang loop unroll(full)
            for (int e = 0; e < 4; ++e) {
              const int j = 4 * g + e;
              v[h] = fmaf(qrow[((j >> 2) * G + h) * 4 + (j & 3)], cb[(mm >> e) & 1], v[h]);
            }
          } else {
#pragma clang loop unroll(full)
            for (int e = 0; e < 2; ++e) {
              const int j = 2 * g + e;
              v[h] = fmaf(qrow[((j >> 2) * G + h) * 4 + (j & 3)], cb[(mm >> (2 * e)) & 3], v[h]);
            }
          }
        }
        sm.t.klut[checked(i, kKeyLutEntries, kCheckDecodeTable)] = make_float4(v[0], v[1], v[2], v[3]);
      }
      widths &= ~6;   // no key quad table
    }
    // pair tables come with the codebook table (a scalar codebook's (c[lo],
    // c[hi]), or PolarQuant's radius-angle pairs); a quad entry is two pairs
    auto stage = [&](int wm, const float* tab, float2* pair, float4* quad, float* cent, bool hilo, const PairSrc& pr) {
      const float2* pt = reinterpret_cast<const float2*>(tab + kPairOffset);
      if (prefetched) {
        // the sources loaded before the scan: every width of 1-4 bits in one
        // pass of the block's threads
        if ((wm >> 4) & 1) {
          const int o = pair_offset(4);
          if (hilo)
            reinterpret_cast<uint2*>(pair)[o + tid] = split_half2(pr.p4.x * kKeyPairScale, pr.p4.y * kKeyPairScale);
          else
            pair[o + tid] = pr.p4;
        }
        if (((wm >> 3) & 1) && tid < 64) {
          const int o = pair_offset(3);
          if (hilo)
            reinterpret_cast<uint2*>(pair)[o + tid] = split_half2(pr.p3.x * kKeyPairScale, pr.p3.y * kKeyPairScale);
          else
            pair[o + tid] = pr.p3;
        }
        if ((wm >> 2) & 1) quad[quad_offset(2) + tid] = make_float4(pr.q2a.x, pr.q2a.y, pr.q2b.x, pr.q2b.y);
        if (((wm >> 1) & 1) && tid < 16) quad[quad_offset(1) + tid] = make_float4(pr.q1a.x, pr.q1a.y, pr.q1b.x, pr.q1b.y);
        wm &= ~0x1E;
      }
      for (int bb = 3; bb <= 4; ++bb) {
        if (!((wm >> bb) & 1)) continue;
        const int o = pair_offset(bb), n = 1 << (2 * bb);
        if (hilo) {
          for (int i = tid; i < n; i += blockDim.x)
            reinterpret_cast<uint2*>(pair)[o + i] = split_half2(pt[o + i].x * kKeyPairScale,
                                                                pt[o + i].y * kKeyPairScale);
        } else {
          for (int i = tid; i < n; i += blockDim.x) pair[o + i] = pt[o + i];
        }
      }
      for (int bb = 1; bb <= 2; ++bb) {
        if (!((wm >> bb) & 1)) continue;
        const int sh = 2 * bb, po = pair_offset(bb), n = 1 << (2 * sh);
        for (int i = tid; i < n; i += blockDim.x) {
          const float2 c0 = pt[po + (i & ((1 << sh) - 1))], c1 = pt[po + (i >> sh)];
          quad[quad_offset(bb) + i] = make_float4(c0.x, c0.y, c1.x, c1.y);
        }
      }
      for (int bb = 5; bb <= 8; ++bb) {
        if (!((wm >> bb) & 1)) continue;
        const int o = centroid_offset(bb), n = 1 << bb;
        for (int i = tid; i < n; i += blockDim.x) cent[o + i] = tab[o + i];
      }
    };
    stage(widths & 0x1FF, a.k_table, sm.t.kpair, sm.t.kquad, sm.t.kcent, key_mfma, pre[0]);
    stage(widths >> 9, a.v_table, sm.t.vpair, sm.t.vquad, sm.t.vcent, false, pre[1]);
    __syncthreads();
    // keep the scheduler from moving table work into the page loop (it
    // otherwise inflates the loop's register use)
    __builtin_amdgcn_sched_barrier(0);
  };
  stage_tables();

  // The other class's own launch keeps the QJL term's table (qjl_scores_lut):
  // 32 x 16 x G floats built once per workgroup from the prepared S q.  The
  // merged launches, whose LDS is sized for 4 waves per SIMD, keep the
  // per-coordinate form (qjl_scores).
  float* qlut = nullptr;
  if constexpr (CLASS == 2) {
    constexpr int kLut = TQ_JL_DIM / 4 * 16 * G;
    __shared__ __align__(16) float lut[kLut];
    qlut = lut;
    if (a.qjl_s != nullptr) {
      const float* qsv = qrow + 2 * D * G;
      for (int idx = tid; idx < kLut; idx += blockDim.x) {
        const int h = idx % G, v = (idx / G) & 15, n = idx / (16 * G);
        const float* c = qsv + (n * G + h) * 4;
        float sum = 0.f;
#pragma clang loop unroll(full)
        for (int e = 0; e < 4; ++e) sum += ((v >> e) & 1) ? c[e] : -c[e];
        lut[idx] = sum;
      }
    }
    __syncthreads();
  }

  // acc: packed pages' value sums on the matrix cores (value_mfma), in the
  // rotated domain; acco: fp16 pages' (classes with fp16 pages), in the
  // original domain until the end
  constexpr int NG = G > 4 ? G / 4 : 1;
  constexpr bool kFp16 = CLASS == 2 || CLASS == 4;
  float m[G], l[G];
  v4f acc[NG][2], acco[kFp16 ? NG : 1][2];
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
  }
#pragma clang loop unroll(full)
  for (int g = 0; g < NG; ++g) acc[g][0] = acc[g][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma clang loop unroll(full)
  for (int g = 0; g < (kFp16 ? NG : 1); ++g) acco[g][0] = acco[g][1] = v4f{0.f, 0.f, 0.f, 0.f};
  float* wv = sm.w[wave];
  if constexpr (G < 4) {
    for (int i = lane; i < 4 * kWRow; i += 64) wv[i] = 0.f;
    wave_lds_sync();
  }

  // The page loop, compiled for page class PC.  The merged launch runs a
  // common-class and a wide-class copy side by side (a uniform branch), each
  // with its own code; it is held to 4 waves per SIMD (a few spills in the
  // wide copy, cheaper than a fourth of the waves).
  auto page_loop = [&](auto pc_tag) {
    constexpr int PC = decltype(pc_tag)::value;
    // sum over coordinates of the QJL query term, per head (lane l adds
    // coordinates 2l and 2l + 1, then a wavefront sum)
    float qsum[G];
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h) qsum[h] = 0.f;
    if (PC == 2 && CLASS != 2 && a.qjl_s != nullptr) {
      const float* qsv = qrow + 2 * D * G;
      const int i0 = 2 * lane;
#pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) {
        const float* c = qsv + ((i0 >> 2) * G + h) * 4 + (i0 & 3);
        qsum[h] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_sum(c[0] + c[1]))));
      }
    }
    // One page's softmax step, shared by the loops below: masks the lanes past
    // the session's tokens, updates the running maximum and sums, writes the
    // page mass, rescales the value sums when the reference moved, and leaves
    // the page's weights (times the value norms) in the wave's LDS rows.
    auto weigh = [&](int p, float (&s)[G], float nv, int valid) {
      float alpha[G];
  #pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h)
        if (lane >= valid) s[h] = -INFINITY;
      // token weights: the scores (log2 units); the combine normalises them
      if constexpr (MASS) {
        if (a.tmass) {
          const size_t ts = (size_t)a.max_pages * PT;
          float* trow = a.tmass + ((size_t)b * a.n_q_heads + hq0) * ts + (size_t)p * PT + lane;
  #pragma clang loop unroll(full)
          for (int h = 0; h < G; ++h) trow[h * ts] = s[h];
        }
      }
      softmax_update<G>(s, m, l, alpha);
      if constexpr (MASS) {
        if (a.mass) {
          float* mrow = a.mass + ((size_t)b * a.n_q_heads + hq0) * a.max_pages + p;
  #pragma clang loop unroll(full)
          for (int h = 0; h < G; ++h) {
            const float ps = wave_sum(s[h]);
            if (lane == 0) mrow[(size_t)h * a.max_pages] = ps > 0.f ? m[h] + log2f(ps) : -INFINITY;
          }
        }
      }
      // the running sums need rescaling only when some head's maximum moved
      // (alpha is wave-uniform, so is the branch)
      bool moved = false;
  #pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) moved |= alpha[h] != 1.f;
      if (moved) {
  #pragma clang loop unroll(full)
        for (int g = 0; g < NG; ++g)
  #pragma clang loop unroll(full)
          for (int i = 0; i < 4; ++i)
            if (4 * g + i < G) {
              acc[g][0][i] *= alpha[4 * g + i];
              acc[g][1][i] *= alpha[4 * g + i];
            }
        if constexpr (kFp16) {
  #pragma clang loop unroll(full)
          for (int g = 0; g < NG; ++g)
  #pragma clang loop unroll(full)
            for (int i = 0; i < 4; ++i)
              if (4 * g + i < G) {
                acco[g][0][i] *= alpha[4 * g + i];
                acco[g][1][i] *= alpha[4 * g + i];
              }
        }
      }
  #pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) wv[h * kWRow + lane] = s[h] * nv;
      wave_lds_sync();
    };

    if constexpr (PC == 0) {
      // Common pages.  Every lane issues the same loads per page (words past
      // a width repeat its last word), K and V together at the page's start,
      // so the V words arrive while the scores are computed; the other waves
      // of the SIMD cover the wait for the K words.
      for (int p = p_begin + wave; p < p_end; p += kDecodeWaves) {
        const PageDesc pd = read_desc(sm.desc[checked(p - p_begin, kMaxPagesPerSplit, kCheckDecodeIndex)]);
        const bool ok = pd.present && !pd.qjl && pd.kb >= 1 && pd.kb <= 4 && pd.vb >= 1 && pd.vb <= 4 &&
                        pd.off + page_size_dev(pd.kb, pd.vb, false) <= a.pool_bytes;
        if (!__builtin_amdgcn_readfirstlane(ok)) continue;
        const int kb = __builtin_amdgcn_readfirstlane(pd.kb), vb = __builtin_amdgcn_readfirstlane(pd.vb);
        const char* kp = a.pool + pd.off;
        const char* vp = kp + 1024 * kb + 256;
        const uint4* ks = reinterpret_cast<const uint4*>(kp);
        const uint4* vs = reinterpret_cast<const uint4*>(vp);
        uint32_t kw[16], vw[16];
        // 3- and 4-bit keys on the matrix cores (every such page of the range
        // set key_mfma when the tables were staged)
        const bool mk = kMfmaKeys && kb >= 3;
        if (mk) {
          (void)checked((int)!key_mfma, 1, kCheckDecodeTable);
          if (kb == 3) load_keys_mfma<3>(kp, lane, kw);
          else load_keys_mfma<4>(kp, lane, kw);
        } else {
  #pragma clang loop unroll(full)
          for (int w = 0; w < 4; ++w) {
            const uint4 x = ks[min(w, kb - 1) * 64 + lane];
            kw[4 * w] = x.x; kw[4 * w + 1] = x.y; kw[4 * w + 2] = x.z; kw[4 * w + 3] = x.w;
          }
        }
        const float nk = reinterpret_cast<const float*>(kp + 1024 * kb)[lane];
  #pragma clang loop unroll(full)
        for (int w = 0; w < 4; ++w) {
          const uint4 y = vs[min(w, vb - 1) * 64 + lane];
          vw[4 * w] = y.x; vw[4 * w + 1] = y.y; vw[4 * w + 2] = y.z; vw[4 * w + 3] = y.w;
        }
        const float nv = reinterpret_cast<const float*>(vp + 1024 * vb)[lane];
        float s[G];
        switch (kb) {
          case 1:
            if (key_table_bits == 1) key_scores_table<1, G>(kw, sm.t.klut, s);
            else key_scores_w<1, G>(kw, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s);
            break;
          case 2:
            if (key_table_bits == 2) key_scores_table<2, G>(kw, sm.t.klut, s);
            else key_scores_w<2, G>(kw, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s);
            break;
          case 3:
            if constexpr (kMfmaKeys)
              key_scores_mfma<3>(kw, lane, sm.t.kqa, reinterpret_cast<const uint2*>(sm.t.kpair) + pair_offset(3), s);
            else
              key_scores_w<3, G>(kw, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s);
            break;
          default:
            if constexpr (kMfmaKeys)
              key_scores_mfma<4>(kw, lane, sm.t.kqa, reinterpret_cast<const uint2*>(sm.t.kpair) + pair_offset(4), s);
            else
              key_scores_w<4, G>(kw, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s);
            break;
        }
        const float ks_scale = mk ? nk * key_unscale : nk;
  #pragma clang loop unroll(full)
        for (int h = 0; h < G; ++h) s[h] *= ks_scale;
        weigh(p, s, nv, min(PT, ntok - p * PT));
        switch (vb) {
          case 1: value_mfma_w<1, NG>(vw, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          case 2: value_mfma_w<2, NG>(vw, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          case 3: value_mfma_w<3, NG>(vw, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          default: value_mfma_w<4, NG>(vw, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
        }
        wave_lds_sync();
      }
      return;
    }

    for (int p = p_begin + wave; p < p_end; p += kDecodeWaves) {
      const PageDesc pd = read_desc(sm.desc[checked(p - p_begin, kMaxPagesPerSplit, kCheckDecodeIndex)]);
      const int kb = pd.kb, vb = pd.vb;
      const bool qjl = pd.qjl;
      const uint64_t off = pd.off;
      if (!pd.present || off + page_size_dev(kb, vb, qjl) > a.pool_bytes) continue;
      if (kb == 0 ? (vb != 0 || qjl) : (kb > 8 || vb < 1 || vb > 8)) continue;
      if (qjl && a.qjl_s == nullptr) continue;
      if (page_class(kb, vb, qjl) != PC) continue;
      if (PC != 0 && ((a.k_polar && kb > 4) || (a.v_polar && vb > 4))) continue;   // no polar pair table
      const char* page = a.pool + off;
      const int valid = min(PT, ntok - p * PT);
      float s[G];
      const char* vblk = page + 1024 * kb + 256;
      // the norms (and the QJL scale) are loaded with the codes, not after them
      float nk = 1.f, nv = 1.f, gq = 0.f;
      if (kb != 0) {
        nk = reinterpret_cast<const float*>(page + 1024 * kb)[lane];
        const char* vb0 = vblk + (qjl ? 1280 : 0);
        nv = reinterpret_cast<const float*>(vb0 + 1024 * vb)[lane];
        if (PC == 2 && qjl) gq = reinterpret_cast<const float*>(vblk + 1024)[lane];
      }
      if (PC == 2 && kb == 0) {
        key_scores_fp16<G>(page, lane, qrow + D * G, s);
      } else {
        if constexpr (PC == 0) {
          switch (kb) {
            case 1: key_scores<1, G>(page, lane, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s); break;
            case 2: key_scores<2, G>(page, lane, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s); break;
            case 3: key_scores<3, G>(page, lane, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s); break;
            default: key_scores<4, G>(page, lane, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s); break;
          }
        } else if constexpr (PC == 1) {
          switch (kb) {
            case 5: key_scores_wide<5, G>(page, lane, qrow, sm.t.kcent, s); break;
            case 6: key_scores_wide<6, G>(page, lane, qrow, sm.t.kcent, s); break;
            case 7: key_scores_wide<7, G>(page, lane, qrow, sm.t.kcent, s); break;
            default: key_scores_wide<8, G>(page, lane, qrow, sm.t.kcent, s); break;
          }
        } else {
          switch (kb) {
            case 1: key_scores<1, G>(page, lane, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s); break;
            case 2: key_scores<2, G>(page, lane, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s); break;
            case 3: key_scores<3, G>(page, lane, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s); break;
            case 4: key_scores<4, G>(page, lane, qrow, sm.t.kpair, sm.t.kquad, sm.t.kcent, s); break;
            case 5: key_scores_wide<5, G>(page, lane, qrow, sm.t.kcent, s); break;
            case 6: key_scores_wide<6, G>(page, lane, qrow, sm.t.kcent, s); break;
            case 7: key_scores_wide<7, G>(page, lane, qrow, sm.t.kcent, s); break;
            default: key_scores_wide<8, G>(page, lane, qrow, sm.t.kcent, s); break;
          }
        }
  #pragma clang loop unroll(full)
        for (int h = 0; h < G; ++h) s[h] *= nk;
        if (PC == 2 && qjl) {
          float t[G];
          if constexpr (CLASS == 2)
            qjl_scores_lut<G>(vblk, lane, qlut, t);
          else
            qjl_scores<G>(vblk, lane, qrow + 2 * D * G, qsum, t);
  #pragma clang loop unroll(full)
          for (int h = 0; h < G; ++h) s[h] = fmaf(gq, t[h], s[h]);
          vblk += 1280;
        }
      }
      weigh(p, s, nv, valid);
      if (PC == 2 && kb == 0) {
        if constexpr (kFp16) value_mfma_fp16<NG>(page, lane, wv, acco);
      } else if constexpr (PC == 0) {
        switch (vb) {
          case 1: value_mfma<1, NG>(vblk, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          case 2: value_mfma<2, NG>(vblk, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          case 3: value_mfma<3, NG>(vblk, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          default: value_mfma<4, NG>(vblk, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
        }
      } else if constexpr (PC == 1) {
        switch (vb) {
          case 5: value_mfma_wide<5, NG>(vblk, lane, wv, sm.t.vcent, acc); break;
          case 6: value_mfma_wide<6, NG>(vblk, lane, wv, sm.t.vcent, acc); break;
          case 7: value_mfma_wide<7, NG>(vblk, lane, wv, sm.t.vcent, acc); break;
          default: value_mfma_wide<8, NG>(vblk, lane, wv, sm.t.vcent, acc); break;
        }
      } else {
        switch (vb) {
          case 1: value_mfma<1, NG>(vblk, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          case 2: value_mfma<2, NG>(vblk, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          case 3: value_mfma<3, NG>(vblk, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          case 4: value_mfma<4, NG>(vblk, lane, wv, sm.t.vpair, sm.t.vquad, acc); break;
          case 5: value_mfma_wide<5, NG>(vblk, lane, wv, sm.t.vcent, acc); break;
          case 6: value_mfma_wide<6, NG>(vblk, lane, wv, sm.t.vcent, acc); break;
          case 7: value_mfma_wide<7, NG>(vblk, lane, wv, sm.t.vcent, acc); break;
          default: value_mfma_wide<8, NG>(vblk, lane, wv, sm.t.vcent, acc); break;
        }
      }
      wave_lds_sync();
    }
  };
  if constexpr (CLASS == 3) {
    if (cls == 0)
      page_loop(std::integral_constant<int, 0>{});
    else
      page_loop(std::integral_constant<int, 1>{});
  } else if constexpr (CLASS == 4) {
    if (cls == 0)
      page_loop(std::integral_constant<int, 0>{});
    else if (cls == 1)
      page_loop(std::integral_constant<int, 1>{});
    else
      page_loop(std::integral_constant<int, 2>{});
  } else {
    page_loop(std::integral_constant<int, CLASS>{});
  }


  // ---- workgroup reduction: waves, then token quarters.
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) l[h] = wave_sum(l[h]);
  if (lane == 0) {
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h) {
      sm.stat[wave][0][h] = m[h];
      sm.stat[wave][1][h] = l[h];
    }
  }
  __syncthreads();
  float M[G];
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) {
    M[h] = -INFINITY;
    for (int w = 0; w < kDecodeWaves; ++w) M[h] = fmaxf(M[h], sm.stat[w][0][h]);
  }
  if (tid < G) {
    const int h = tid;
    float lsum = 0.f;
    for (int w = 0; w < kDecodeWaves; ++w)
      if (sm.stat[w][0][h] != -INFINITY) lsum += sm.stat[w][1][h] * exp2f(sm.stat[w][0][h] - M[h]);
    float* ph = part + h * head_stride;
    ph[0] = M[h];
    ph[1] = lsum;
  }
  float fsc[G];
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) fsc[h] = m[h] == -INFINITY ? 0.f : exp2f(m[h] - M[h]);
  // the fp16 pages' sums join the rotated-domain sums
  if constexpr (kFp16) add_rotated<NG>(acco, lane, a.sign_mask, acc);
  // the matrix-core sums: lane L holds coordinates v_stream_coord(L, 0 / 1)
  {
    const int c0 = v_stream_coord(lane, 0), c1 = v_stream_coord(lane, 1);
#pragma clang loop unroll(full)
    for (int g = 0; g < NG; ++g)
#pragma clang loop unroll(full)
      for (int i = 0; i < 4; ++i)
        if (4 * g + i < G) {
          sm.red[wave][(4 * g + i) * D + c0] = acc[g][0][i] * fsc[4 * g + i];
          sm.red[wave][(4 * g + i) * D + c1] = acc[g][1][i] * fsc[4 * g + i];
        }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    float v = 0.f;
#pragma clang loop unroll(full)
    for (int w = 0; w < kDecodeWaves; ++w) v += sm.red[w][idx];
    const int h = idx / D, j = idx - h * D;
    part[h * head_stride + 4 + j] = v;
  }
}

// (3) combine: one 128-thread block per (session, query head).  The split
// weights 2^(m_s - M) are computed once into LDS; the value sums then stream
// with independent loads.
constexpr int kCombineGroups = 4;                  // 128-thread groups per row
constexpr int kCombineWaves = kCombineGroups * 2;

// Merges the partials of one (session, query head) row: log-sum-exp weights,
// a compacted list of the non-empty partials (ascending, so the sum order is
// fixed), their value sums split over four thread groups, then one FWHT.
__global__ __launch_bounds__(128 * kCombineGroups) void combine_kernel(DecodeArgs a) {
  __shared__ float wgt[kMaxPartials];
  __shared__ int list[kMaxPartials];
  __shared__ float gsum[kCombineGroups][D];
  __shared__ float red[kCombineWaves];
  __shared__ int cnt[kCombineWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = 128 * kCombineGroups;
  const int row = blockIdx.x;
  const int b = row / a.n_q_heads;
  const int ns = a.n_partials;   // every class that ran
  const float* part = a.wsp + (size_t)row * ns * kPartialFloats;
  float* o = a.out + (size_t)row * D;
  // the classes whose split launch left this row's unit out: their partials
  // were never written and count as empty
  const int unit = b * a.n_kv_heads + (row - b * a.n_q_heads) / a.group;
  int skip = 0;
  if (unit < TQ_MAX_LISTED_UNITS) {
#pragma clang loop unroll(full)
    for (int c = 0; c < 3; ++c) skip |= (int)((a.unit_skip[c][unit >> 5] >> (unit & 31)) & 1u) << c;
  }
  auto m_of = [&](int s) {
    const int c = s < a.part_base[1] ? 0 : s < a.part_base[2] ? 1 : 2;
    return (skip >> c) & 1 ? -INFINITY : part[(size_t)s * kPartialFloats];
  };
  // global max over partials
  float mloc = -INFINITY;
  for (int s = tid; s < ns; s += nthr) mloc = fmaxf(mloc, m_of(s));
  mloc = wave_max(mloc);
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  float M = red[0];
#pragma clang loop unroll(full)
  for (int w = 1; w < kCombineWaves; ++w) M = fmaxf(M, red[w]);
  float* mrow = a.mass ? a.mass + (size_t)row * a.max_pages : nullptr;
  float* trow = a.tmass ? a.tmass + (size_t)row * a.max_pages * PT : nullptr;
  if (M == -INFINITY || a.n_tokens[b] <= 0) {
    if (tid < D) o[tid] = 0.f;
    if (mrow)
      for (int p = tid; p < a.max_pages; p += nthr) mrow[p] = 0.f;
    if (trow)
      for (int t = tid; t < a.max_pages * PT; t += nthr) trow[t] = 0.f;
    return;
  }
  // weights, the denominator and the list of non-empty partials
  int total = 0;
  for (int base = 0; base < ns; base += nthr) {
    const int s = base + tid;
    float f = 0.f;
    if (s < ns) {
      const float ms = m_of(s);
      f = ms == -INFINITY ? 0.f : exp2f(ms - M);
      wgt[s] = f;
    }
    const uint64_t bal = __ballot(f != 0.f);
    __syncthreads();                               // red / cnt free again
    if (lane == 0) cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = total, all = total;
#pragma clang loop unroll(full)
    for (int w = 0; w < kCombineWaves; ++w) {
      off += w < wave ? cnt[w] : 0;
      all += cnt[w];
    }
    if (f != 0.f) list[checked(off + (int)__popcll(bal & ((1ull << lane) - 1ull)), kMaxPartials, kCheckCombine)] = s;
    total = all;
  }
  __syncthreads();
  // the denominator, summed over the list in rank order, so that the result
  // does not depend on where the partials sit (which classes ran)
  float lloc = 0.f;
  for (int k = tid; k < total; k += nthr) {
    const int s = checked(list[k], ns, kCheckCombine);
    lloc = fmaf(part[(size_t)s * kPartialFloats + 1], wgt[s], lloc);
  }
  lloc = wave_sum(lloc);
  __syncthreads();
  if (lane == 0) red[wave] = lloc;
  __syncthreads();
  float L = 0.f;
#pragma clang loop unroll(full)
  for (int w = 0; w < kCombineWaves; ++w) L += red[w];
  if (mrow) {
    const float invL = 1.0f / L;
    for (int p = tid; p < a.max_pages; p += nthr) {
      const float v = mrow[p];
      mrow[p] = v == -INFINITY ? 0.f : exp2f(v - M) * invL;
    }
  }
  if (trow) {
    const float invL = 1.0f / L;
    float4* t4 = reinterpret_cast<float4*>(trow);
    for (int i = tid; i < a.max_pages * PT / 4; i += nthr) {
      float4 v = t4[i];
      v.x = v.x == -INFINITY ? 0.f : exp2f(v.x - M) * invL;
      v.y = v.y == -INFINITY ? 0.f : exp2f(v.y - M) * invL;
      v.z = v.z == -INFINITY ? 0.f : exp2f(v.z - M) * invL;
      v.w = v.w == -INFINITY ? 0.f : exp2f(v.w - M) * invL;
      t4[i] = v;
    }
  }
  // value sums: group g takes list entries g, g + 4, ...; four loads in flight
  const int g = tid >> 7, j = tid & (D - 1);
  float acc4[4] = {0.f, 0.f, 0.f, 0.f};
  int k = g;
  for (; k + 3 * kCombineGroups < total; k += 4 * kCombineGroups) {
#pragma clang loop unroll(full)
    for (int u = 0; u < 4; ++u) {
      const int s = list[k + u * kCombineGroups];
      acc4[u] = fmaf(part[(size_t)s * kPartialFloats + 4 + j], wgt[s], acc4[u]);
    }
  }
  for (; k < total; k += kCombineGroups) {
    const int s = list[k];
    acc4[0] = fmaf(part[(size_t)s * kPartialFloats + 4 + j], wgt[s], acc4[0]);
  }
  gsum[g][j] = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
  __syncthreads();
  // o = D H D acc / d / L; the transform exchanges through gsum[0] (thread j
  // alone reads column j of gsum, before it writes gsum[0][j])
  uint32_t neg = 0;
  float ar = 0.f;
  if (tid < D) {
#pragma clang loop unroll(full)
    for (int q = 0; q < kCombineGroups; ++q) ar += gsum[q][j];
    neg = (a.sign_mask[j >> 5] >> (j & 31)) & 1u;
  }
  const float hv = fwht128_two_waves(flip_if(ar, neg), j, tid < D, gsum[0]);
  if (tid < D) o[j] = flip_if(hv, neg) * (1.0f / D) / L;
}


}  // namespace
}  // namespace dev
}  // namespace tq

using namespace tq;
using namespace tq::dev;

int tq::check_word_decode(uint32_t* out, bool reset) { return read_check_word(out, reset); }

namespace {

template <int CLASS, bool MASS>
void launch_split(int G, dim3 grid, dim3 blk, hipStream_t s, const DecodeArgs& a, const uint64_t* pages,
                  const UnitList& l) {
  switch (G) {
    case 1: hipLaunchKernelGGL((split_kernel<1, CLASS, MASS>), grid, blk, 0, s, a, a.wsq, pages, a.wsp, l); break;
    case 2: hipLaunchKernelGGL((split_kernel<2, CLASS, MASS>), grid, blk, 0, s, a, a.wsq, pages, a.wsp, l); break;
    case 4: hipLaunchKernelGGL((split_kernel<4, CLASS, MASS>), grid, blk, 0, s, a, a.wsq, pages, a.wsp, l); break;
    default:
      // the merged launches (CLASS 3, 4) are not used for groups of 8
      if constexpr (CLASS < 3)
        hipLaunchKernelGGL((split_kernel<8, CLASS, MASS>), grid, blk, 0, s, a, a.wsq, pages, a.wsp, l);
      break;
  }
}

template <int CLASS>
void launch_split_any(bool mass, int G, dim3 grid, dim3 blk, hipStream_t s, const DecodeArgs& a,
                      const uint64_t* pages, const UnitList& l) {
  if (mass)
    launch_split<CLASS, true>(G, grid, blk, s, a, pages, l);
  else
    launch_split<CLASS, false>(G, grid, blk, s, a, pages, l);
}

int decode_impl(const tq_layer* layer, const tq_cache* cache, const tq_query* query, float* out,
                float* page_mass, float* token_mass, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!query || !query->q) return fail(TQ_ERR_INVALID_ARG, "null query");
  if (query->dtype != TQ_DTYPE_F16 && query->dtype != TQ_DTYPE_F32)
    return fail(TQ_ERR_INVALID_ARG, "unknown query dtype %d", query->dtype);
  if (query->n_q_heads <= 0 || query->n_q_heads % cache->n_kv_heads)
    return fail(TQ_ERR_INVALID_ARG, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                query->n_q_heads, cache->n_kv_heads);
  const int G = query->n_q_heads / cache->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(TQ_ERR_UNSUPPORTED, "GQA group %d not in {1, 2, 4, 8}", G);
  if (query->stride_b < 0 || query->stride_h < 0) return fail(TQ_ERR_INVALID_ARG, "negative stride");
  if (!out || !workspace) return fail(TQ_ERR_INVALID_ARG, "null output or workspace");
  if (!aligned16(out) || !aligned16(workspace)) return fail(TQ_ERR_ALIGNMENT, "out/workspace misaligned");
  if (((uintptr_t)page_mass & 3) != 0) return fail(TQ_ERR_ALIGNMENT, "page_mass misaligned");
  if (((uintptr_t)token_mass & 15) != 0) return fail(TQ_ERR_ALIGNMENT, "token_mass misaligned");
  if (!(query->softmax_scale >= 0.f) || isinf(query->softmax_scale))
    return fail(TQ_ERR_INVALID_ARG, "bad softmax scale");
  if (query->qjl_scoring != TQ_QJL_SCORE_UNBIASED && query->qjl_scoring != TQ_QJL_SCORE_SIGN)
    return fail(TQ_ERR_INVALID_ARG, "unknown qjl_scoring %d", query->qjl_scoring);
  SplitPlan sp = split_plan(cache->n_sessions, cache->n_kv_heads, cache->max_pages);
  const int max_partials = sp.n_splits + sp.max_splits_wide + sp.n_splits_general;
  if (max_partials > kMaxPartials)   // the combine stages their weights in LDS
    return fail(TQ_ERR_UNSUPPORTED, "%d partials per row exceed %d", max_partials, kMaxPartials);
  const size_t need = decode_workspace_bytes(cache->n_sessions, query->n_q_heads, sp);
  if (workspace_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  DecodeArgs a;
  a.q = query->q;
  a.q_dtype = query->dtype;
  a.q_sb = query->stride_b;
  a.q_sh = query->stride_h;
  a.n_q_heads = query->n_q_heads;
  a.group = G;
  const float scale = query->softmax_scale > 0.f ? query->softmax_scale : 0.08838834764831845f;
  a.scale2 = scale * kLog2e;
  a.qjl_sign = query->qjl_scoring == TQ_QJL_SCORE_SIGN;
  a.k_polar = layer->k_codebook == TQ_CODEBOOK_POLAR;
  a.v_polar = layer->v_codebook == TQ_CODEBOOK_POLAR;
  a.n_tokens = cache->n_tokens;
  a.n_sessions = cache->n_sessions;
  a.n_kv_heads = cache->n_kv_heads;
  a.max_pages = cache->max_pages;
  a.pool = reinterpret_cast<const char*>(cache->pool);
  a.pool_bytes = cache->pool_bytes;
  a.sign_mask = layer->sign_mask;
  a.k_table = layer->k_table;
  a.v_table = layer->v_table;
  a.qjl_s = layer->qjl_s;
  // A page class the host says is absent gets no launch and no partials.
  const int cls = cache->page_classes == 0
                      ? (TQ_CACHE_COMMON_PAGES | TQ_CACHE_WIDE_PAGES | TQ_CACHE_OTHER_PAGES)
                      : cache->page_classes;
  const bool run_common = (cls & TQ_CACHE_COMMON_PAGES) != 0;
  const bool run_wide = (cls & TQ_CACHE_WIDE_PAGES) != 0;
  const bool run_other = (cls & TQ_CACHE_OTHER_PAGES) != 0;
  // Per-class unit lists from the host's per-unit record: a class's launch
  // covers only the units that hold it.  Class 0 = common, 1 = wide, 2 = other.
  UnitList lists[3];
  const int class_bit[3] = {TQ_CACHE_COMMON_PAGES, TQ_CACHE_WIDE_PAGES, TQ_CACHE_OTHER_PAGES};
  const int64_t units = (int64_t)cache->n_sessions * cache->n_kv_heads;
  const bool listed = cache->unit_classes != nullptr && units <= TQ_MAX_LISTED_UNITS;
  std::memset(a.unit_skip, 0, sizeof(a.unit_skip));
  for (int c = 0; c < 3; ++c) {
    lists[c].n = 0;
    lists[c].group[0] = lists[c].group[1] = lists[c].group[2] = 0;
    if (!listed) continue;
    for (int u = 0; u < (int)units; ++u) {
      if (cache->unit_classes[u] & class_bit[c])
        lists[c].unit[lists[c].n++] = (uint16_t)u;
      else
        a.unit_skip[c][u >> 5] |= 1u << (u & 31);
    }
  }
  // one grid row per listed unit, else (H_kv, B) over every unit
  auto grid_of = [&](int n_splits, const UnitList& l) {
    return listed ? dim3(n_splits, l.n, 1) : dim3(n_splits, cache->n_kv_heads, cache->n_sessions);
  };
  const dim3 blk(64 * kDecodeWaves);
  const bool go_common = run_common && (!listed || lists[0].n > 0);
  const bool go_wide = run_wide && (!listed || lists[1].n > 0);
  const bool go_other = run_other && (!listed || lists[2].n > 0);
  // Beside common pages, the wide class and the other class (sink and tail
  // pages, a minority there) join one merged launch; a layer without common
  // pages (QJL or fp16 alone, say) keeps each class's own kernel.
  const int cnt[3] = {listed ? lists[0].n : (int)units, listed ? lists[1].n : (int)units,
                      listed ? lists[2].n : (int)units};
  // (groups of 8 query heads keep separate launches: the merged kernel does
  // not fit 4 waves per SIMD at that width)
  const bool merge = G <= 4 && go_common;
  const bool merge_other = merge && go_other &&
                           (!listed || cnt[0] + (go_wide ? cnt[1] : 0) + cnt[2] <= 2 * TQ_MAX_LISTED_UNITS);
  // A merged launch of common and wide pages (listed units, ranges not cut
  // for a long context; the other class's blocks, mostly empty ranges around
  // a decode loop's tail pages, are not counted) balances its ranges: wide ranges shorter in proportion to a wide page's
  // cost (whole pages per wave), common ones the shortest that keep the
  // launch within one round of kTargetSplitGroups workgroups.
  int lc = sp.pages_per_split, lw = sp.pages_per_split_wide;
  if (listed && merge && go_wide && !sp.cut) {
    const int M = cache->max_pages, lmax = std::min(M, kMaxPagesPerSplit);
    for (int l = sp.pages_per_split; l <= lmax; ++l) {
      const int per_wave = (l + kDecodeWaves - 1) / kDecodeWaves;
      const int w = std::min(l, std::max(sp.min_pages_per_split_wide,
                                         kDecodeWaves * std::max(1, (int)(per_wave / kWidePageCost))));
      lc = l;
      lw = w;
      const int64_t groups = (int64_t)cnt[0] * ((M + l - 1) / l) + (int64_t)cnt[1] * ((M + w - 1) / w);
      if (groups <= kTargetSplitGroups) break;
    }
  }
  // short contexts: the other class's middle ranges after the common ones
  a.other_edges_first = !sp.cut;
  a.n_splits = (cache->max_pages + lc - 1) / lc;
  a.pages_per_split = lc;
  a.n_splits_general = sp.n_splits_general;
  a.pages_per_split_general = sp.pages_per_split_general;
  a.n_splits_wide = (cache->max_pages + lw - 1) / lw;
  a.pages_per_split_wide = lw;
  const int n_common = run_common ? a.n_splits : 0;
  const int n_wide = run_wide ? a.n_splits_wide : 0;
  const int n_other = run_other ? sp.n_splits_general : 0;
  a.part_base[0] = 0;
  a.part_base[1] = n_common;
  a.part_base[2] = n_common + n_wide;
  a.n_partials = n_common + n_wide + n_other;
  a.wsq = reinterpret_cast<float*>(workspace);
  a.wsp = a.wsq + (size_t)cache->n_sessions * query->n_q_heads * kQPrepFloats;
  a.out = out;
  a.mass = page_mass;
  a.tmass = token_mass;
  const bool mass = page_mass != nullptr || token_mass != nullptr;
  hipStream_t s = (hipStream_t)stream;
  const int rows = cache->n_sessions * query->n_q_heads;
  hipLaunchKernelGGL(qprep_kernel, dim3(rows), dim3(128), 0, s, a);
  if ((st = launch_status("query prep"))) return st;
  if (merge && (go_wide || merge_other)) {
    UnitList merged;
    merged.n = 0;
    merged.group[2] = merge_other ? cnt[2] : 0;
    merged.group[1] = go_wide ? cnt[1] : 0;
    merged.group[0] = cnt[0];
    if (listed) {
      for (int c = 2; c >= 0; --c)
        for (int i = 0; i < merged.group[c]; ++i) merged.unit[merged.n++] = lists[c].unit[i];
    }
    const int64_t blocks = (int64_t)merged.group[2] * a.n_splits_general +
                           (int64_t)merged.group[1] * a.n_splits_wide + (int64_t)merged.group[0] * a.n_splits;
    if (merge_other)
      launch_split_any<4>(mass, G, dim3((unsigned)blocks), blk, s, a, cache->pages, merged);
    else
      launch_split_any<3>(mass, G, dim3((unsigned)blocks), blk, s, a, cache->pages, merged);
    if ((st = launch_status("split (merged classes)"))) return st;
  } else if (go_common) {
    launch_split_any<0>(mass, G, grid_of(a.n_splits, lists[0]), blk, s, a, cache->pages, lists[0]);
    if ((st = launch_status("split (common pages)"))) return st;
  } else if (go_wide) {
    launch_split_any<1>(mass, G, grid_of(a.n_splits_wide, lists[1]), blk, s, a, cache->pages, lists[1]);
    if ((st = launch_status("split (wide pages)"))) return st;
  }
  if (go_other && !merge_other) {
    launch_split_any<2>(mass, G, grid_of(a.n_splits_general, lists[2]), blk, s, a, cache->pages, lists[2]);
    if ((st = launch_status("split (other pages)"))) return st;
  }
  hipLaunchKernelGGL(combine_kernel, dim3(rows), dim3(128 * kCombineGroups), 0, s, a);
  return launch_status("combine");
}

// Device scratch of tq_decode_attention_noalloc: the query-prep rows and the
// split partials, in a file-scope device array (one copy per GPU, allocated
// with the code object and held until the process ends) in place of a caller's
// workspace.
constexpr size_t kScratchBytes = TQ_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kScratchBytes];

// The device address of `scratch` on the current device, looked up once per
// device.  In host code the array's name is only a host-side stand-in, never a
// device address.
int scratch_address(void** out) {
  static std::atomic<void*> cached[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(TQ_ERR_UNSUPPORTED, "device %d: at most 64 devices", dev);
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(TQ_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    cached[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return ok();
}

}  // namespace

extern "C" {

int tq_device_checks(uint32_t* flags, int reset) {
  if (!flags) return fail(TQ_ERR_INVALID_ARG, "null flags");
  *flags = 0;
#if TQ_DEVICE_CHECKS
  int st;
  if ((st = check_word_encode(flags, reset)) || (st = check_word_pages(flags, reset)) ||
      (st = check_word_decode(flags, reset)) || (st = check_word_dequant(flags, reset)))
    return fail(st, "reading the device check words failed");
  return ok();
#else
  (void)reset;
  return fail(TQ_ERR_UNSUPPORTED, "a release build has no device checks");
#endif
}

int tq_decode_attention_noalloc(const tq_layer* layer, const tq_cache* cache, const tq_query* query,
                                float* out, void* stream) {
  if (!cache || !query) return fail(TQ_ERR_INVALID_ARG, "null cache or query");
  const size_t need = tq_decode_workspace_bytes(cache, query->n_q_heads);
  if (need == 0) return fail(TQ_ERR_INVALID_ARG, "invalid cache or query-head count");
  if (need > kScratchBytes)
    return fail(TQ_ERR_WORKSPACE, "decode needs %zu bytes of scratch; the built-in scratch holds %zu",
                need, kScratchBytes);
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st) return st;
  return decode_impl(layer, cache, query, out, nullptr, nullptr, ws, kScratchBytes, stream);
}

int tq_decode_attention(const tq_layer* layer, const tq_cache* cache, const tq_query* query,
                        float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(layer, cache, query, out, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int tq_decode_attention_mass(const tq_layer* layer, const tq_cache* cache, const tq_query* query,
                             float* out, float* page_mass, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!page_mass) return fail(TQ_ERR_INVALID_ARG, "null page_mass");
  return decode_impl(layer, cache, query, out, page_mass, nullptr, workspace, workspace_bytes, stream);
}

int tq_decode_attention_token_mass(const tq_layer* layer, const tq_cache* cache, const tq_query* query,
                                   float* out, float* token_mass, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!token_mass) return fail(TQ_ERR_INVALID_ARG, "null token_mass");
  return decode_impl(layer, cache, query, out, nullptr, token_mass, workspace, workspace_bytes, stream);
}

}  // extern "C"
