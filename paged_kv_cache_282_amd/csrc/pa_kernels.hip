// Device code of libpa: KV append, block copy, paged decode and chunked-prefill
// attention for CDNA4 (gfx950, wave64).
//
// What is computed follows the pages:
//   * "Module 4 · Batching, Scheduling, and Paging", section "PagedAttention":
//     K/V live in fixed-size blocks reached through a per-sequence block table;
//     the kernels gather through that indirection. Section "Block sharing":
//     shared blocks are copied on the first divergent write.
//   * worksonmygpu.com continuous-batching post, section "Selective batching":
//     each request attends over its own tokens, softmax(q K^T * scale) V;
//     section "The prefill/decode mix": prefill chunks in the same iteration.
//
// How it is computed is this file's own design for gfx950:
//   * Decode works on items (sequence, kv head, 1024-token partition) that a
//     persistent grid takes from a queue; a workgroup's four waves take
//     interleaved 32-token steps of an item, keep an online softmax state
//     each and merge in LDS. A sequence of several partitions gets one
//     partial per partition, which the persistent kernel folds into the
//     sequence's output itself (log-sum-exp identity); only the fallback for
//     batches of more than 2048 sequences leaves them to a second kernel. The
//     grid size and the loads' cache policy follow the batch.
//   * bf16 decode: scores and p.V run on v_mfma_f32_16x16x32_bf16, whose 16
//     columns are the query heads of one GQA group (padded); bf16 prefill runs
//     on v_mfma_f32_32x32x16_bf16, whose 32 columns are (position, head) rows.
//     The pool keeps K in 8-element slices and V in 4-token slices, so every
//     MFMA operand is one contiguous load (decode) or LDS read (prefill), and
//     each lane's scores are exactly the tokens whose V values the same lane
//     holds for p.V: probabilities never leave registers. Every load
//     instruction reads a single block through a uniform base address
//     (decode: a buffer descriptor of one kv head's K or V tile).
//   * Tokens outside a context are excluded by selection (-inf scores, zeroed
//     V), never by multiplying with p = 0, so NaN in unused slots is harmless.
//   * fp32: a VALU kernel with the same work decomposition (16 lanes per token
//     for q.K, dimension-owning lanes for p.V).
#include "pa_launch.h"

#include <stdint.h>

#include <mutex>
#include <type_traits>

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ constexpr bf16x2 kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

// Block-table entry read through the scalar cache (the row pointer and index
// are wave-uniform; the tables are not written while a kernel runs). Scalar
// loads are counted apart from vector loads, so waiting for a table entry
// never waits for KV loads issued earlier.
typedef const __attribute__((address_space(4))) int32_t* table_ptr;
__device__ __forceinline__ int table_entry(const int32_t* row, int idx) {
  return ((table_ptr)row)[idx];  // address-space cast
}

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Four floats as a float vector. (Reading float lanes out of an integer vector
// with __builtin_bit_cast on a vector element is avoided on purpose: clang
// lowers that to a read of element 0.)
__device__ __forceinline__ f32x4 ld16f(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// Buffer descriptor of `bytes` bytes from `base` (raw: no stride, byte
// offsets; out-of-range reads return zero). 0x00020000 is the descriptor's
// format word for untyped 32-bit data on this target.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}
// Cache-policy bits of a buffer load: the default (cached), or nt
// (nontemporal: streamed past the caches).
constexpr int kCached = 0;
constexpr int kNontemporal = 2;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of scores that are never NaN (tokens a row may not see are set to
// -inf first, and slots outside a context are never scored unmasked). The
// NaN-propagating maximum lowers to v_maximum3_f32 as it stands; the IEEE
// maxNum of fmaxf needs a quieting v_max of every operand first.
__device__ __forceinline__ float smax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float smax8(const float (&x)[8]) {
  return smax(smax(smax(smax(x[0], x[1]), x[2]), smax(smax(x[3], x[4]), x[5])),
              smax(x[6], x[7]));
}

// Max / sum over the four 16-lane groups (lanes l, l^16, l^32, l^48).
// Maximum over the four 16-lane rows of the wave at each lane position: swap
// halves, then neighbouring rows, with the cross-lane VALU permutes.
__device__ __forceinline__ float max_over_groups(float x) {
  // (vector elements are read by value: bit casts of an element expression
  // have read element 0)
  const uint32_t u = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = smax(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const uint32_t v = __float_as_uint(x);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return smax(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
// Sum over the 16 lanes of a group; every lane receives the total.
__device__ __forceinline__ float sum_over_row16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x + __shfl_xor(x, 8);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// Four consecutive values as one store: 16 bytes of float or 8 of bf16.
template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, f32x4 v) {
  u32x2 w;
  w[0] = f32_to_bf16_bits(v[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
  w[1] = f32_to_bf16_bits(v[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
  *reinterpret_cast<u32x2*>(p) = w;
}
template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
               __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
}

__device__ __forceinline__ int clamp_block(int blk, int64_t nb) {
  return (static_cast<uint32_t>(blk) < static_cast<uint64_t>(nb)) ? blk : 0;
}

// ---------------------------------------------------------------------------
// bf16 decode MFMA engine: online-softmax attention of NT column tiles of 16
// query rows over 32-token steps of one kv head (every kernel here uses one
// tile, NT = 1).
//
// A step is 32 tokens: set a = tokens 0..15, set b = tokens 16..31 (two
// blocks of 16, or the two halves of one block of 32).
// Lane (kg = lane/16, r = lane%16):
//   score MFMA  S^T[tok][row] = K[tok][:] . Q[row][:]
//     A (K)  lane gives slice 4s+kg of token r of the set (16 contiguous bytes;
//            a quarter-wave reads 256 contiguous bytes)
//     B (Q)  lane gives Q[row r][32s + 8kg .. +7]
//     C      lane (kg, n) gets tokens 4kg+i of set a and of set b, i < 4.
//   p.V MFMA   O^T[dim][row] += V^T[dim][tok] . P^T[tok][row]
//     A (V^T) lane gives dim 16j + r at tokens 4kg..4kg+3 of set a and of set
//             b: two 8-byte 4-token slices
//     B (P)   lane gives row n at the same eight tokens (its own scores)
//     C       lane (kg, n) holds O^T[16j + 4kg + i][n], i < 4.
// ---------------------------------------------------------------------------
// How far (in base-2 exponent) the running maximum may pass the reference
// maximum before the softmax state is rescaled; weights stay below 2^8.
constexpr float kRescaleSlack = 8.f;
constexpr float kSlackWeight = 256.f;  // 2^kRescaleSlack
// The reference maximum of a row that has seen no key yet: finite, so that
// exp2(s - m) needs no special case before the first key (it is 0 for every
// masked score), and a state with l = 0 adds nothing wherever states merge.
constexpr float kNoMax = -0x1.0p100f;

template <int D, int BS, int NT>
struct Bf16Engine {
  static constexpr int KS = D / 32;
  static constexpr int VT = D / 16;
  bf16x8 qreg[NT][KS];
  f32x4 o[NT][VT];
  float m[NT], l[NT];
  int lim[NT];  // last token this lane's row may attend to (-1: none)

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m[nt] = kNoMax;
      l[nt] = 0.f;
      lim[nt] = -1;
#pragma unroll
      for (int j = 0; j < VT; ++j) o[nt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) qreg[nt][s] = bf16x8{};
    }
  }

  // Load row `nt`'s query (lane's 8-element slices) from q_row (nullptr: zero).
  __device__ __forceinline__ void load_q(int nt, const uint16_t* q_row, int kg) {
    if (q_row == nullptr) return;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qreg[nt][s] = __builtin_bit_cast(bf16x8, ld16(q_row + 32 * s + 8 * kg));
  }

  // Registers of one 32-token step: K rows of the two score sets and V^T.
  struct KV {
    u32x4 kA[KS], kB[KS], vv[VT];
  };

  // Issue the loads of a 32-token step. Tokens t0..t0+15 live in block blkA
  // and t0+16..t0+31 in blkB (bs 16) or all in blkA (bs 32).
  // POL is the loads' cache policy (kNontemporal or kCached).
  template <int POL = kNontemporal>
  __device__ __forceinline__ void load_kv(KV& kv, const uint16_t* __restrict__ pool,
                                          int64_t blk_elems, int64_t kofs, int64_t vofs, int blkA,
                                          int blkB, int lane, bool live = true) const {
    // A step that will not be computed (live == false) still issues its loads,
    // so that the number of loads in flight is the same on every path, but it
    // reads block 0 and every lane of an instruction reads the same 16 bytes.
    // Each load is a buffer load through a descriptor of one kv head's K or V
    // tile: the tile base is wave-uniform (scalar registers), each lane adds
    // its constant offset and a compile-time displacement, and the hardware
    // returns zero for anything outside the tile. K/V read once are best
    // loaded with the nontemporal hint: streaming them past the caches this
    // way sustains a higher HBM read rate on this chip than plain loads. K/V
    // that other sequences of the batch read too (shared blocks) are loaded
    // cached instead, so those readers find them in the caches.
    const int r = lane & 15, kg = lane >> 4;
    if (!live) blkA = blkB = 0;
    blkA = __builtin_amdgcn_readfirstlane(blkA);
    blkB = __builtin_amdgcn_readfirstlane(blkB);
    const uint16_t* bA = pool + static_cast<int64_t>(blkA) * blk_elems;
    const uint16_t* bB = (BS == 16) ? pool + static_cast<int64_t>(blkB) * blk_elems : bA;
    constexpr int kTile = BS * D * 2;  // bytes of one kv head's K (or V) tile
    const auto kra = tile_rsrc(bA + kofs, kTile), krb = tile_rsrc(bB + kofs, kTile);
    const auto vra = tile_rsrc(bA + vofs, kTile), vrb = tile_rsrc(bB + vofs, kTile);
    // lane's K byte offset (slice kg, token r) and V byte offset (4-token
    // slice kg, dim r); set b of a 32-slot block starts at token 16
    const int ko = live ? (kg * BS + r) * 16 : 0;
    const int vo = live ? (kg * D + r) * 8 : 0;
    constexpr int kb = BS == 16 ? 0 : 16 * 16;     // set b: tokens 16.. of the same K slice
    constexpr int vb = BS == 16 ? 0 : 4 * D * 8;   // set b: 4-token slices 4..7
    constexpr int ks = 4 * BS * 16;  // next 4 slices of K
    constexpr int vs = 16 * 8;       // next 16 dims of V
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kv.kA[s] = __builtin_amdgcn_raw_buffer_load_b128(kra, ko + ks * s, 0, POL);
      kv.kB[s] = __builtin_amdgcn_raw_buffer_load_b128(krb, ko + kb + ks * s, 0, POL);
    }
#pragma unroll
    for (int j = 0; j < VT; ++j) {
      const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(vra, vo + vs * j, 0, POL);
      const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(vrb, vo + vb + vs * j, 0, POL);
      kv.vv[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  }

  // First half of a step: q.k of every tile, from the K operands alone.
  __device__ __forceinline__ void scores(const u32x4 (&kA)[KS], const u32x4 (&kB)[KS],
                                         f32x4 (&sa)[NT], f32x4 (&sb)[NT]) const {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      sa[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      sb[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sa[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kA[s]),
                                                         qreg[nt][s], sa[nt], 0, 0, 0);
        sb[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kB[s]),
                                                         qreg[nt][s], sb[nt], 0, 0, 0);
      }
    }
  }

  // Second half of a step starting at token t0: masks, online softmax and
  // p.V for every tile. With EDGE, tokens >= vend have their V zeroed (they
  // may be NaN) and scores of tokens past a row's limit are -inf, where the
  // step reaches that far; without it the caller guarantees that the whole
  // step lies before vend and at or before every real row's limit.
  template <bool EDGE = true>
  __device__ __forceinline__ void finish(f32x4 (&sa)[NT], f32x4 (&sb)[NT], u32x4 (&vv)[VT],
                                         int t0, int vend, int lane, float sl2e) {
    if constexpr (EDGE) edge_masks(sa, sb, vv, t0, vend, lane);
    softmax_pv(sa, sb, vv, sl2e);
  }

  __device__ __forceinline__ void edge_masks(f32x4 (&sa)[NT], f32x4 (&sb)[NT], u32x4 (&vv)[VT],
                                             int t0, int vend, int lane) {
    const int kg = lane >> 4;
    // element e of this lane's eight tokens: e < 4 -> t0 + 4kg + e (set a),
    // e >= 4 -> t0 + 16 + 4kg + e - 4 (set b)
    const int ta0 = t0 + 4 * kg, tb0 = t0 + 16 + 4 * kg;
    if (t0 + 32 > vend) {  // wave-uniform: zero V of tokens past the end
      const int na = vend - ta0, nb = vend - tb0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int nv = w < 2 ? na : nb;
        const int e0 = 2 * (w & 1);
        const uint32_t mask = (e0 < nv ? 0x0000FFFFu : 0u) | (e0 + 1 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int j = 0; j < VT; ++j) vv[j][w] &= mask;
      }
    }
    // Mask the scores of tokens past a row's limit. Only steps that reach
    // past the limit of some real row need it (one wave-uniform test per
    // step, for every tile at once); then padding rows (lim < 0) are masked
    // entirely, otherwise their scores are finite and are never read.
    bool reach = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) reach = reach || (lim[nt] >= 0 && t0 + 31 > lim[nt]);
    if (__builtin_amdgcn_ballot_w64(reach) != 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sa[nt][i] = (ta0 + i <= lim[nt]) ? sa[nt][i] : -__builtin_inff();
          sb[nt][i] = (tb0 + i <= lim[nt]) ? sb[nt][i] : -__builtin_inff();
        }
      }
    }
  }

  // Online softmax and p.V of every tile, on scores already masked.
  __device__ __forceinline__ void softmax_pv(f32x4 (&sa)[NT], f32x4 (&sb)[NT], u32x4 (&vv)[VT],
                                             float sl2e) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // raw scores q.k; the softmax runs in base 2 on q.k * sl2e
      float sc[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] = sa[nt][i];
        sc[4 + i] = sb[nt][i];
      }
      // scaling by sl2e > 0 is monotone, so the scaled maximum is mx * sl2e.
      // The reference m only moves when the running maximum passes it by more
      // than kRescaleSlack (base 2): until then the weights exp2(s - m) stay
      // below 2^kRescaleSlack, and the state needs no rescale. Any reference
      // gives the same softmax, since O and l share it.
      const float mx = max_over_groups(smax8(sc));
      const float mtop = smax(m[nt], mx * sl2e);
      const bool g = mtop > m[nt] + kRescaleSlack;
      const float mnew = g ? mtop : m[nt];
      bf16x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = static_cast<__bf16>(exp2_fast(fmaf(sc[e], sl2e, -mnew)));
      // the row sum adds the bf16 weights that p.V uses
      float ps = 0.f;
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), kOnes2, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), kOnes2, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), kOnes2, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), kOnes2, ps, false);
      // l and o need rescaling only where a maximum that had seen a key grew
      // (elsewhere alpha is 1, or l and o are still zero): the factor, its
      // exp2 and the products are computed only then
      if (__builtin_amdgcn_ballot_w64(g && m[nt] != kNoMax) != 0) {
        const float alpha = exp2_fast(m[nt] - mnew);
        l[nt] *= alpha;
#pragma unroll
        for (int j = 0; j < VT; ++j) o[nt][j] *= alpha;
      }
      l[nt] += ps;
      m[nt] = mnew;
#pragma unroll
      for (int j = 0; j < VT; ++j)
        o[nt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv[j]),
                                                           p, o[nt][j], 0, 0, 0);
    }
  }

  // A whole loaded step: scores, then softmax and p.V.
  __device__ __forceinline__ void compute(KV& kv, int t0, int vend, int lane, float sl2e) {
    f32x4 sa[NT], sb[NT];
    scores(kv.kA, kv.kB, sa, sb);
    finish(sa, sb, kv.vv, t0, vend, lane, sl2e);
  }

  __device__ __forceinline__ void step(const uint16_t* __restrict__ pool, int64_t blk_elems,
                                       int64_t kofs, int64_t vofs, int blkA, int blkB, int t0,
                                       int vend, int lane, float sl2e) {
    KV kv;
    load_kv(kv, pool, blk_elems, kofs, vofs, blkA, blkB, lane);
    compute(kv, t0, vend, lane, sl2e);
  }
};

// ---------------------------------------------------------------------------
// fp32 VALU engine: G query rows (one GQA group) of one kv head.
// Lane (grp = lane/16, c = lane%16). In a 32-token step, group grp owns tokens
// 8grp .. 8grp+7. q.K: lane holds dims c*EPL .. +EPL of a K row; the 16 lanes
// sum their partial dot products. p.V: lane owns dims c + 16k and reads the
// two 4-token V slices of those 8 tokens.
// ---------------------------------------------------------------------------
template <int D, int BS, int G>
struct F32Engine {
  static constexpr int EPL = D / 16;
  float qv[G][EPL];
  float acc[G][EPL];
  float m[G], l[G];
  int lim;  // last token the rows may attend to (uniform)

  __device__ __forceinline__ void init(const float* q_rows, int c) {
    // q_rows: G consecutive rows of D floats (nullptr: no rows)
#pragma unroll
    for (int qi = 0; qi < G; ++qi) {
      m[qi] = -__builtin_inff();
      l[qi] = 0.f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        acc[qi][k] = 0.f;
        qv[qi][k] = q_rows ? q_rows[qi * D + c * EPL + k] : 0.f;
      }
    }
  }

  __device__ __forceinline__ void step(const float* __restrict__ pool, int64_t blk_elems,
                                       int64_t kofs, int64_t vofs, int blkA, int blkB, int t0,
                                       int vend, int lane, float sl2e) {
    const int grp = lane >> 4, c = lane & 15;
    const float* base;
    int slot0;
    if constexpr (BS == 16) {
      base = pool + static_cast<int64_t>(grp < 2 ? blkA : blkB) * blk_elems;
      slot0 = 8 * (grp & 1);
    } else {
      base = pool + static_cast<int64_t>(blkA) * blk_elems;
      slot0 = 8 * grp;
    }
    const int tbase = t0 + 8 * grp;
    float s[8][G];
    // lane's K dims c*EPL .. +EPL lie in one 8-element slice
    const int kslice = (c * EPL) / 8, ksub = (c * EPL) % 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float* kr = base + kofs + (kslice * BS + slot0 + e) * 8 + ksub;
      float kv[EPL];
#pragma unroll
      for (int k4 = 0; k4 < EPL / 4; ++k4) {
        const f32x4 w = ld16f(kr + 4 * k4);
#pragma unroll
        for (int x = 0; x < 4; ++x) kv[4 * k4 + x] = w[x];
      }
      const bool valid = tbase + e <= lim;
#pragma unroll
      for (int qi = 0; qi < G; ++qi) {
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < EPL; ++k) part = fmaf(kv[k], qv[qi][k], part);
        part = sum_over_row16(part);
        s[e][qi] = valid ? part * sl2e : -__builtin_inff();
      }
    }
#pragma unroll
    for (int qi = 0; qi < G; ++qi) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, s[e][qi]);
      mx = max_over_groups(mx);
      const float mnew = fmaxf(m[qi], mx);
      const float muse = (mnew == -__builtin_inff()) ? 0.f : mnew;
      const float alpha = exp2_fast(m[qi] - muse);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[e][qi] = exp2_fast(s[e][qi] - muse);
        ps += s[e][qi];
      }
      l[qi] = l[qi] * alpha + ps;
      m[qi] = mnew;
#pragma unroll
      for (int k = 0; k < EPL; ++k) acc[qi][k] *= alpha;
    }
    const bool tail = t0 + 32 > vend;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      // dim c + 16k at tokens slot0 .. slot0+7: two 4-token slices
      const float* vr = base + vofs + ((slot0 / 4) * D + c + 16 * k) * 4;
      float v[8];
      const f32x4 w0 = ld16f(vr), w1 = ld16f(vr + D * 4);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        v[x] = w0[x];
        v[4 + x] = w1[x];
      }
      if (tail) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (tbase + e < vend) ? v[e] : 0.f;
      }
#pragma unroll
      for (int qi = 0; qi < G; ++qi)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[qi][k] = fmaf(s[e][qi], v[e], acc[qi][k]);
    }
  }
};

// ---------------------------------------------------------------------------
// Workgroup-level merge of the per-wave states held in LDS.
// ---------------------------------------------------------------------------
constexpr int kMaxGroup = 8;  // query heads per kv head handled by the decode kernels

template <int D, int R = kMaxGroup>
struct MergeSmem {
  float o[kWaves][R][D];
  float m[kWaves][R];
  float l[kWaves][R];
};

// Combines the kWaves states of row `row` at dimensions dd .. dd+3: (M, L, O).
template <int D, int R>
__device__ __forceinline__ void combine_waves(const MergeSmem<D, R>& sm, int row, int dd, float& M,
                                              float& L, f32x4& O) {
  M = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][row]);
  L = 0.f;
  O = f32x4{0.f, 0.f, 0.f, 0.f};
  if (M == -__builtin_inff()) return;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float f = exp2_fast(sm.m[w][row] - M);
    const f32x4 ow = *reinterpret_cast<const f32x4*>(&sm.o[w][row][dd]);
    L = fmaf(sm.l[w][row], f, L);
#pragma unroll
    for (int x = 0; x < 4; ++x) O[x] = fmaf(ow[x], f, O[x]);
  }
}

// Split-K merge of one output row's four dimensions, one partition at a time
// in partition order (the log-sum-exp identity):
//   M' = max(M, M_j),  w = L_j 2^(M_j - M'),  L' = L 2^(M - M') + w,
//   O' = O 2^(M - M') + o_j w,
// where o_j = O_j / L_j is partition j's normalised output exactly as stored
// (rounded to the output type) and the result is O / L. Every path that
// merges partitions -- the persistent decode, which folds each partition as it
// finishes, and the merge kernel, which reads them from the workspace -- folds
// with these operations in this order, so a sequence's bits do not depend on
// which path ran.
struct MergeState {
  float M, L;
  f32x4 O;
  __device__ __forceinline__ void reset() {
    M = -__builtin_inff();
    L = 0.f;
    O = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void fold(float Mj, float Lj, f32x4 oj) {
    const float bm = fmaxf(M, Mj);
    const float f = exp2_fast(M - bm);  // 0 on the first fold (M = -inf)
    const float w = Lj * exp2_fast(Mj - bm);
    L = fmaf(L, f, w);
#pragma unroll
    for (int x = 0; x < 4; ++x) O[x] = fmaf(oj[x], w, O[x] * f);
    M = bm;
  }
  __device__ __forceinline__ f32x4 result() const {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    return O * inv;
  }
};

// A partial output as the merge reads it back: the stored element type's
// value (bf16 rounding, nearest even) as float.
template <typename OutT>
__device__ __forceinline__ f32x4 as_stored(f32x4 v);
template <>
__device__ __forceinline__ f32x4 as_stored<float>(f32x4 v) {
  return v;
}
template <>
__device__ __forceinline__ f32x4 as_stored<uint16_t>(f32x4 v) {
  f32x4 r;
#pragma unroll
  for (int x = 0; x < 4; ++x) r[x] = __uint_as_float(static_cast<uint32_t>(f32_to_bf16_bits(v[x])) << 16);
  return r;
}

// After each wave has written its state: a single-partition sequence stores
// its normalised output; otherwise this partition publishes (M, L, o) for the
// merge kernel, where o = O / L is the partition's own normalised output,
// rounded to the output type like a final row.
//
// Workspace layout: the partials of one (sequence, kv head) item are
// contiguous, partition-major: o at ws_o[(p * rows + row) * D + d] (elements
// of OutT) and (M, L) at ws_ml[(p * rows + row) * 2 + {0, 1}] (float), from
// this (sequence, kv head)'s base. A partition's rows x D partial is one
// contiguous run written with 8- or 16-byte stores. These writes, interleaved
// with the stream of K/V reads, cost several times their bytes in HBM time,
// so a bf16 call keeps its partials in bf16: half the bytes of float.
template <int D, typename OutT>
__device__ __forceinline__ void finish_partition(const MergeSmem<D>& sm, int rows, int np, int p,
                                                 OutT* __restrict__ out_rows,
                                                 OutT* __restrict__ ws_o,
                                                 float* __restrict__ ws_ml) {
  constexpr int C4 = D / 4;
  for (int c = threadIdx.x; c < rows * C4; c += kWaves * 64) {
    const int row = c / C4, dd = 4 * (c - row * C4);
    float M, L;
    f32x4 O;
    combine_waves(sm, row, dd, M, L, O);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (np == 1) {
      store4<OutT>(out_rows + row * D + dd, O * inv);
    } else {
      store4<OutT>(ws_o + (static_cast<int64_t>(p) * rows + row) * D + dd, O * inv);
      if (dd == 0) {
        ws_ml[(static_cast<int64_t>(p) * rows + row) * 2 + 0] = M;
        ws_ml[(static_cast<int64_t>(p) * rows + row) * 2 + 1] = L;
      }
    }
  }
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* pool;
  const int32_t* tables;
  const int32_t* lens;
  int num_seqs, mb, hq, hkv, max_ctx, np_max, n_items;
  int64_t nb, blk_elems;
  float sl2e;
  void* ws_o;  // partial outputs, elements of the output type
  float* ws_ml;
  // Caller's sharing hint (nullptr: none): share[b] leading tokens of sequence
  // b are said to live in the same blocks as sequence b-1's.
  const int32_t* share;
  // Decode step with its append (nullptr: none): k_new / v_new
  // [num_seqs][hkv][D] are the keys and values at position lens[b]-1 of
  // sequence b, written to pool slot slots[b] (negative: not written).
  const void* k_new;
  const void* v_new;
  const int32_t* slots;
};

// Resolves (sequence, kv head, partition) of this workgroup; false if idle.
struct DecodeItem {
  int b, g, p, np, tok0, tok1;
};
// Workgroup -> (sequence, kv head, partition). Items are ordered
// partition-major: every sequence's first partition comes first, then every
// second partition, and so on. Each item is at most one partition long, so
// the hardware dispatcher balances them; the grid is sized for the longest
// context and items past a sequence's last partition exit at once, in the
// trailing part of the grid.
template <int BS>
__device__ __forceinline__ bool decode_item(const DecodeArgs& a, DecodeItem& it) {
  const int item = blockIdx.x;
  if (item >= a.n_items) return false;
  const int groups = a.num_seqs * a.hkv;
  it.p = item / groups;
  const int bg = item - it.p * groups;
  it.b = bg / a.hkv;
  it.g = bg - it.b * a.hkv;
  int n = a.lens[it.b];
  n = n < 0 ? 0 : n;
  n = n > a.max_ctx ? a.max_ctx : n;
  n = n > a.mb * BS ? a.mb * BS : n;
  it.np = n > 0 ? (n + kPartition - 1) / kPartition : 1;
  if (it.p >= it.np) return false;
  it.tok0 = it.p * kPartition;
  it.tok1 = min(n, it.tok0 + kPartition);
  return true;
}

template <int BS>
__device__ __forceinline__ void step_blocks(const int32_t* __restrict__ trow, int t0, int vend,
                                            int64_t nb, int& blkA, int& blkB) {
  if constexpr (BS == 16) {
    blkA = trow[t0 >> 4];
    blkB = (t0 + 16 < vend) ? trow[(t0 >> 4) + 1] : blkA;
  } else {
    blkA = trow[t0 >> 5];
    blkB = blkA;
  }
  blkA = clamp_block(blkA, nb);
  blkB = clamp_block(blkB, nb);
}

template <int D, int BS>
__global__ __launch_bounds__(256) void decode_bf16_kernel(DecodeArgs a) {
  DecodeItem it;
  if (!decode_item<BS>(a, it)) return;
  __shared__ MergeSmem<D> sm;
  const int G = a.hq / a.hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, kg = lane >> 4;
  const uint16_t* pool = static_cast<const uint16_t*>(a.pool);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);

  Bf16Engine<D, BS, 1> eng;
  eng.init();
  if (r < G) {
    eng.load_q(0, q + (static_cast<int64_t>(it.b) * a.hq + it.g * G + r) * D, kg);
    eng.lim[0] = it.tok1 - 1;
  }
  const int64_t kofs = static_cast<int64_t>(it.g) * BS * D;
  const int64_t vofs = static_cast<int64_t>(a.hkv) * BS * D + static_cast<int64_t>(it.g) * D * BS;
  const int32_t* trow = a.tables + static_cast<int64_t>(it.b) * a.mb;
  for (int t0 = it.tok0 + wave * kStep; t0 < it.tok1; t0 += kWaves * kStep) {
    int blkA, blkB;
    step_blocks<BS>(trow, t0, it.tok1, a.nb, blkA, blkB);
    eng.step(pool, a.blk_elems, kofs, vofs, blkA, blkB, t0, it.tok1, lane, a.sl2e);
  }
  const float lt = sum_over_groups(eng.l[0]);
  if (r < G) {
    if (kg == 0) {
      sm.m[wave][r] = eng.m[0];
      sm.l[wave][r] = lt;
    }
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
      *reinterpret_cast<f32x4*>(&sm.o[wave][r][16 * j + 4 * kg]) = eng.o[0][j];
  }
  __syncthreads();

  const int64_t row0 = static_cast<int64_t>(it.b) * a.hq + it.g * G;
  finish_partition<D, uint16_t>(sm, G, it.np, it.p,
                                static_cast<uint16_t*>(a.out) + row0 * D,
                                static_cast<uint16_t*>(a.ws_o) + row0 * a.np_max * D,
                                a.ws_ml + row0 * a.np_max * 2);
}

// ---------------------------------------------------------------------------
// Persistent bf16 decode with a dynamic work queue (batches of up to
// kMaxScanSeqs sequences).
//
// The unit of work is a whole (sequence, kv head): one workgroup computes its
// partitions one after another and folds each partition's partial result
// into the row's merge state in registers as soon as the partition is done
// (MergeState: the same operations, in the same order, as the merge kernel
// applies to partials read back from the workspace), so no partial result
// goes through memory and no merge launch follows.
//
// Every workgroup first scans the context lengths into LDS and ranks the
// sequences into ordering classes, longest first: more partitions first,
// then single-partition sequences by length in 128-token classes (sequence
// order inside a class). Units are numbered in that order, the kv heads of a
// sequence next to each other, so the queue ends with the shortest units and
// the last units of every workgroup are short. Workgroups take units from an
// atomic counter in the workspace until it runs past the last one; the last
// workgroup to leave returns the counters to zero for the next call. Nothing
// waits on another workgroup.
// ---------------------------------------------------------------------------
constexpr int kMaxScanSeqs = 2048;
constexpr int kOrderClasses = 16;  // ordering classes of the sequences (see order_class)

struct ScanSmem {
  int n[kMaxScanSeqs];      // clamped context length
  // Units in queue order: the sequence index (bits 0..10). A unit that
  // stacks the members of a shared prefix (see decode_loop) also holds its
  // member count - 1 (bits 11..14) and its shared partitions (bits 16..31).
  int order[kMaxScanSeqs];
  int wsum[kOrderClasses / 4 + 1][kWaves][2];  // one scratch row per block scan
  int ccount[kWaves][kOrderClasses];           // units per wave and class (one sequence per thread)
  unsigned long long tokens;  // sum of the clamped context lengths
  int shared;                 // some sequence starts with its predecessor's first block
  int units;                  // number of units per kv head
};
static_assert(kMaxScanSeqs <= 2048, "a unit entry keeps the sequence index in 11 bits");

// Rows of MFMA columns a unit of stacked members fills: up to 16 / G members
// of G query heads each.
constexpr int kStackRows = 16;

// A context length as the kernels use it: at least 0, at most max_ctx and at
// most what the table row can address.
template <int BS>
__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int n) {
  n = n < 0 ? 0 : n;
  n = n > a.max_ctx ? a.max_ctx : n;
  return n > a.mb * BS ? a.mb * BS : n;
}

// Partitions of a context of n tokens (an empty context is one empty item).
__device__ __forceinline__ int partitions_of(int n) {
  return n > 0 ? (n + kPartition - 1) / kPartition : 1;
}

// Ordering class of a sequence: 8 + (partitions - 1), at most 15, for
// sequences of several partitions; for single-partition sequences its length
// in 128-token classes (0 .. 7). Larger classes come first.
__device__ __forceinline__ int order_class(int n) {
  const int np = partitions_of(n);
  return np >= 2 ? min(kOrderClasses - 1, 7 + np) : min(7, n / (kPartition / 8));
}

// Exclusive block-wide maximum (256 threads, -1 before thread 0) of values x
// that are -1 or grow with the thread index: the nearest lower thread's x that
// is not -1. Scratch is one row of ScanSmem::wsum, which no other scan of the
// same call uses.
__device__ __forceinline__ int block_last_excl(int (&wsum)[kWaves][2], int x) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __builtin_amdgcn_ballot_w64(x >= 0);
  if (lane == 0) wsum[wave][0] = m != 0 ? __builtin_amdgcn_readlane(x, 63 - __builtin_clzll(m)) : -1;
  const uint64_t below = m & ((1ull << lane) - 1);
  const int inw = __shfl(x, below != 0 ? 63 - __builtin_clzll(below) : 0);
  __syncthreads();
  int b = -1;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    if (w < wave) b = max(b, wsum[w][0]);
  return below != 0 ? inw : b;
}

// Exclusive block-wide scan (256 threads) of a pair of counts; scratch is one
// row of ScanSmem::wsum, which no other scan of the same call uses.
__device__ __forceinline__ void block_scan2(int (&wsum)[kWaves][2], int x, int y, int& ex,
                                            int& ey, int& tx, int& ty) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ix = x, iy = y;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int ox = __shfl_up(ix, d), oy = __shfl_up(iy, d);
    if (lane >= d) {
      ix += ox;
      iy += oy;
    }
  }
  if (lane == 63) {
    wsum[wave][0] = ix;
    wsum[wave][1] = iy;
  }
  __syncthreads();
  int bx = 0, by = 0;
  tx = 0;
  ty = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) {
      bx += wsum[w][0];
      by += wsum[w][1];
    }
    tx += wsum[w][0];
    ty += wsum[w][1];
  }
  ex = bx + ix - x;
  ey = by + iy - y;
}

// One queue item: partition p of unit (sequence b, kv head g) and its token
// range; np is the sequence's number of partitions.
struct QItem {
  int unit, b, g, p, np, tok0, tok1;
  // units that stack shared-prefix members only: the first member b0, the
  // member count, the shared partitions S, this item's member m (own
  // partitions p >= S), and whether it is a shared partition (all members)
  int b0, ucnt, S, m, stacked;
};

// An item is the same for the whole workgroup; say so, so that everything
// derived from it lives in scalar registers.
__device__ __forceinline__ void make_uniform(QItem& it) {
  it.unit = __builtin_amdgcn_readfirstlane(it.unit);
  it.b = __builtin_amdgcn_readfirstlane(it.b);
  it.g = __builtin_amdgcn_readfirstlane(it.g);
  it.p = __builtin_amdgcn_readfirstlane(it.p);
  it.np = __builtin_amdgcn_readfirstlane(it.np);
  it.tok0 = __builtin_amdgcn_readfirstlane(it.tok0);
  it.tok1 = __builtin_amdgcn_readfirstlane(it.tok1);
}
__device__ __forceinline__ void make_uniform_stack(QItem& it) {
  it.b0 = __builtin_amdgcn_readfirstlane(it.b0);
  it.ucnt = __builtin_amdgcn_readfirstlane(it.ucnt);
  it.S = __builtin_amdgcn_readfirstlane(it.S);
  it.m = __builtin_amdgcn_readfirstlane(it.m);
  it.stacked = __builtin_amdgcn_readfirstlane(it.stacked);
}

// Items are processed as a pipeline. While item i computes, every wave already
// holds the block ids and query of item i+1, and as soon as a wave finishes
// its steps of item i it issues the first two steps of item i+1, so the
// workgroup barrier and the fold of item i overlap memory traffic of item i+1.
//
// Every load of the step pipeline is issued unconditionally, in straight-line
// code: a step past the end of its item (or a prefetch past the end of the
// queue) reads block 0, which stays cached, and is never computed. Loads
// inside branches would make the compiler's wait counts conservative (wait for
// all outstanding loads), which serialises loads and compute.
template <int D, int R = kMaxGroup>
struct DecodeSmem {
  MergeSmem<D, R> sm2[2];  // wave states of consecutive items alternate
  ScanSmem sc;
  int s_next[2];
  int s_ok[2][kWaves];  // stacked items: every member's blocks match (per wave)
};

// The queue counters live at the start of the decode workspace: [0] the next
// decode unit, [1] workgroups that have left, [2] the next prefill tile of a
// mixed launch. The last workgroup to leave returns them to zero.
__device__ __forceinline__ void leave_queue(int32_t* __restrict__ queue) {
  if (threadIdx.x == 0) {
    const int done = atomicAdd(&queue[1], 1);
    if (done == static_cast<int>(gridDim.x) - 1) {  // everyone else has left
      atomicExch(&queue[0], 0);
      atomicExch(&queue[2], 0);
      atomicExch(&queue[1], 0);
    }
  }
}

// K+V bytes of a call up to which its loads stay cached: a batch this small
// may still be in the 256 MiB last-level cache when it is read again.
constexpr uint64_t kCachedCallBytes = 256ull << 20;

// Every workgroup scans the context lengths into LDS and ranks the sequences
// into unit order. Returns whether the call's
// K/V loads should stay cached: when some sequence's first block is also its
// predecessor's (parallel samples or a cached prefix: the blocks are read
// again by the other sequences), or when the call reads little enough for the
// caches to hold it.
//
// SH (a sharing hint is given): a run of consecutive sequences each of which
// declares that its first partitions live in its predecessor's blocks is cut
// into stacks of up to kStackRows / G members. A stack whose members all have
// at least one partition of their own after S >= 1 shared ones becomes one
// unit (entered under its first member, with the member count and S); its
// members enter no unit of their own. The declaration is only used to form
// stacks: decode_loop checks every shared block id before relying on it.
template <int D, int BS, bool SH, int R>
__device__ __forceinline__ bool decode_scan(const DecodeArgs& a, int32_t* __restrict__ queue,
                                            DecodeSmem<D, R>& ds) {
  ScanSmem& sc = ds.sc;
  const int B = a.num_seqs;
  constexpr int kPer = kMaxScanSeqs / 256;
  const int per = (B + 255) / 256;  // thread t owns sequences t*per .. t*per+per-1
  int nl[kPer], cls[kPer], val[kPer];
  int claim[kPer];  // SH: shared partitions declared with the predecessor
  int shared = 0;
  uint64_t tok = 0;
  {
    // The first table entries are loaded together with the lengths (never
    // behind them), so the scan waits for one round trip to memory.
    int first[kPer], before[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int i = threadIdx.x * per + c;
      nl[c] = 0;
      first[c] = -1;
      before[c] = -2;
      claim[c] = 0;
      if (c < per && i < B) {
        nl[c] = a.lens[i];
        first[c] = a.tables[static_cast<int64_t>(i) * a.mb];
        if (i > 0) before[c] = a.tables[static_cast<int64_t>(i - 1) * a.mb];
        if (SH && i > 0) claim[c] = a.share[i];
      }
    }
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int i = threadIdx.x * per + c;
      cls[c] = -1;
      val[c] = i;
      if (c < per && i < B) {
        nl[c] = clamp_len<BS>(a, nl[c]);
        cls[c] = order_class(nl[c]);
        tok += static_cast<uint64_t>(nl[c]);
        shared |= (nl[c] > 0 && first[c] == before[c] &&
                   static_cast<uint32_t>(first[c]) < static_cast<uint64_t>(a.nb)) ? 1 : 0;
        // whole partitions of the declared tokens, leaving this sequence at
        // least one partition of its own
        claim[c] = claim[c] > 0 ? min(claim[c] / kPartition, partitions_of(nl[c]) - 1) : 0;
      }
    }
  }
  if constexpr (SH) {
    // The lengths and claims go to LDS (the order array serves as scratch
    // until the ranking below overwrites it), so that each thread can see
    // its neighbours'.
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int i = threadIdx.x * per + c;
      if (c < per && i < B) {
        sc.n[i] = nl[c];
        sc.order[i] = claim[c];
      }
    }
    __syncthreads();
    // A claim also needs the predecessor to have a partition of its own after
    // the shared ones; a sequence without a valid claim starts a run.
    auto link = [&](int j) {  // shared partitions of sequence j with j - 1 (0: starts a run)
      return j > 0 ? max(0, min(sc.order[j], partitions_of(sc.n[j - 1]) - 1)) : 0;
    };
    int last_start = -1;
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int i = threadIdx.x * per + c;
      if (c < per && i < B && link(i) == 0) last_start = i;
    }
    int run = block_last_excl(sc.wsum[kOrderClasses / 4], last_start);
    const int G = a.hq / a.hkv;
    const int gmax = max(1, kStackRows / G);
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int i = threadIdx.x * per + c;
      if (!(c < per && i < B)) continue;
      if (link(i) == 0) run = i;
      // this sequence's stack: lead .. lead+cnt-1, the run cut every gmax members
      const int lead = i - (i - run) % gmax;
      int cnt = 1, S = partitions_of(sc.n[lead]) - 1;
      int64_t total = sc.n[lead];
      for (int j = lead + 1; j < min(B, lead + gmax); ++j) {
        const int lj = link(j);
        if (lj == 0) break;
        ++cnt;
        S = min(S, lj);
        total += sc.n[j];
      }
      if (cnt >= 2 && S >= 1) {
        S = min(S, 0xFFFF);
        if (i == lead) {
          // one unit: the shared partitions once, then every member's own
          const int64_t work = total - static_cast<int64_t>(cnt - 1) * S * kPartition;
          cls[c] = order_class(static_cast<int>(min<int64_t>(work, 0x7FFFFFFF)));
          val[c] = i | ((cnt - 1) << 11) | (S << 16);
          shared = 1;
        } else {
          cls[c] = -1;  // computed inside its stack's unit
        }
      }
    }
  }
  // Rank the units: by class, largest first, and by sequence index within a
  // class. pos[c] is unit c's place in the order.
  if (threadIdx.x == 0) {
    sc.tokens = 0;
    sc.shared = 0;
  }
  int pos[kPer];
#pragma unroll
  for (int c = 0; c < kPer; ++c) pos[c] = 0;
  if (per == 1) {
    // One sequence per thread: a ballot per class gives each unit its rank
    // among the units of its class in lower lanes, and each wave's count.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int rank = 0, wc = 0;
#pragma unroll
    for (int k = 0; k < kOrderClasses; ++k) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(cls[0] == k);
      if (cls[0] == k)
        rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                         __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
      if (lane == k) wc = __builtin_popcountll(m);
    }
    if (lane < kOrderClasses) sc.ccount[wave][lane] = wc;
    __syncthreads();  // (also orders the clears above)
    // the unit's place: the units of every larger class, then those of its
    // class in lower waves, then in lower lanes
    int units = 0;
    pos[0] = rank;
#pragma unroll
    for (int k = kOrderClasses - 1; k >= 0; --k) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int c = sc.ccount[w][k];
        units += c;
        pos[0] += (k > cls[0] || (k == cls[0] && w < wave)) ? c : 0;
      }
    }
    if (threadIdx.x == 0) sc.units = units;
  } else {
    // Count this thread's units per class, two 16-bit counts per word (a
    // count never exceeds kMaxScanSeqs < 2^16), and scan the counts over the
    // block: each class's start in the order, and this thread's offset in it.
    int cnt[kOrderClasses / 2];
#pragma unroll
    for (int k = 0; k < kOrderClasses / 2; ++k) cnt[k] = 0;
#pragma unroll
    for (int c = 0; c < kPer; ++c)
      if (cls[c] >= 0) cnt[cls[c] >> 1] += 1 << (16 * (cls[c] & 1));
    int ex[kOrderClasses / 2], tot[kOrderClasses / 2];
#pragma unroll
    for (int k = 0; k < kOrderClasses / 2; k += 2)  // (the first barrier also orders the clears)
      block_scan2(sc.wsum[k / 2], cnt[k], cnt[k + 1], ex[k], ex[k + 1], tot[k], tot[k + 1]);
    // class starts, largest class first
    int start[kOrderClasses];
    int run = 0;
#pragma unroll
    for (int k = kOrderClasses - 1; k >= 0; --k) {
      start[k] = run;
      run += (tot[k >> 1] >> (16 * (k & 1))) & 0xFFFF;
    }
    if (threadIdx.x == 0) sc.units = run;
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      int p = 0, before_here = 0;
#pragma unroll
      for (int k = 0; k < kOrderClasses; ++k)
        if (k == cls[c]) p = start[k] + ((ex[k >> 1] >> (16 * (k & 1))) & 0xFFFF);
#pragma unroll
      for (int c2 = 0; c2 < kPer; ++c2)
        before_here += (c2 < c && cls[c2] == cls[c]) ? 1 : 0;
      pos[c] = p + before_here;
    }
  }
  if (tok != 0) atomicAdd(&sc.tokens, static_cast<unsigned long long>(tok));
  if (shared) atomicOr(&sc.shared, 1);
#pragma unroll
  for (int c = 0; c < kPer; ++c) {
    const int i = threadIdx.x * per + c;
    if (cls[c] >= 0) sc.order[pos[c]] = val[c];
    if (c < per && i < B) sc.n[i] = nl[c];
  }
  __syncthreads();
  const uint64_t bytes = sc.tokens * static_cast<uint64_t>(a.hkv) * 2 * D * 2;
  return __builtin_amdgcn_readfirstlane(sc.shared != 0 || bytes <= kCachedCallBytes) != 0;
}

// The decode pipeline of one workgroup after the scan: takes units until the
// queue runs past the last one. POL is the cache policy of the K/V loads.
//
// Units are dealt, not raced for, at the start: of the `dealt` workgroups
// that start together, the one of rank r takes units r and 2*dealt-1-r (it
// needs two: the one it computes and the next one, planned ahead), so the
// longest units, which come first, go one to a workgroup, and the longest of
// the second round goes with the shortest of the first (a batch of about
// two units per workgroup ends up balanced); every further unit comes from
// the queue counter, numbered from 2 * dealt. A workgroup that joins later
// (rank < 0) takes both of its first units from the counter.
//
// SH: a unit may stack the members b0 .. b0+ucnt-1 of a shared prefix (see
// decode_scan). Its first S items are the shared partitions, computed once
// for every member at once: member k's G query rows fill MFMA columns
// kG .. kG+G-1, and the K/V come through b0's table. MFMA columns and the
// softmax of each row are independent, so every row's partial is the one
// its own sequence would compute. Those partials go to the workspace; then
// each member's own partitions follow, and a member folds the stored shared
// partials, in partition order, before its first own one: the same
// operations in the same order as for an unstacked sequence, so the results
// are bit-identical. A shared item's block ids are checked against every
// member's table when it is planned; if any differs, that item and the
// rest of the unit run unstacked instead (b0's item is the same work).
//
// HANDOVER: a wave hands over to the next item as soon as its own steps of the
// current one are done (below); this needs more registers than two
// workgroups per compute unit leave, so the mixed launch runs without it.
//
// FUSED: each sequence's new token (k_new, v_new) is its key and value at
// position lens[b]-1. The wave whose step reads that position replaces the
// token's K and V in the step's registers with them, which is what the step
// would have loaded had the token been appended first; the pool itself is
// written by the kernel itself (append_load, append_store).
template <int D, int BS, int POL, bool SH = false, int R = kMaxGroup, bool HANDOVER = false,
          bool FUSED = false>
__device__ __forceinline__ void decode_loop(const DecodeArgs& a, int32_t* __restrict__ queue,
                                            DecodeSmem<D, R>& ds, int rank, int dealt) {
  using Eng = Bf16Engine<D, BS, 1>;
  constexpr int KS = Eng::KS;
  constexpr int C4 = D / 4;
  constexpr int kSteps = kPartition / (kWaves * kStep);  // steps per wave per partition
  static_assert(kSteps % 2 == 0, "steps alternate between two register buffers");
  static_assert(kMaxGroup * C4 <= kWaves * 64, "one thread per (row, 4 dimensions) of a unit");
  static_assert(!SH || R >= kStackRows, "stacked units need a wave-state row per MFMA column");
  static_assert(2 * kSteps == 16, "a member's block ids of one wave fill 16 lanes");
  MergeSmem<D, R>(&sm2)[2] = ds.sm2;
  ScanSmem& sc = ds.sc;
  int(&s_next)[2] = ds.s_next;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, kg = lane >> 4;
  const int G = a.hq / a.hkv;
  const uint16_t* pool = static_cast<const uint16_t*>(a.pool);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const int total = (SH ? sc.units : a.num_seqs) * a.hkv;  // units

  // Block ids of this wave's steps (0 for steps past the item's end) and the
  // query slices of one item. An item is planned one item ahead; its table
  // entries (lanes 0 .. 2*kSteps-1 load one each) and query slices are loaded
  // then but read only when its first loads are issued, after the current
  // item's third step has been waited for. Vector loads complete in order, so
  // by then those reads wait for nothing; reading them at once would wait for
  // every KV load issued before them.
  struct Plan {
    QItem it;
    int ent;  // lane l < 2*kSteps: table entry of step l/2, block A (l even) or B
    int idA[kSteps], idB[kSteps];
    // SH, shared items: lane l's entry of member 4k + l/16, for the check
    int entm[kStackRows / 4];
    bool ok;  // SH: this wave's block ids are every member's
    // FUSED: the new token's position (-1: not in this item), K slice
    // lane % (D/8) of its row and V dimensions 2 lane, 2 lane + 1 (the patch
    // gathers each lane's parts from these with lane shuffles)
    int pn;
    u32x4 knew;
    uint32_t vnew;
  };
  // rows of MFMA columns an item's results occupy
  auto rows_of = [&](const QItem& it) { return (SH && it.stacked) ? it.ucnt * G : G; };
  // m, S: SH only -- the member and, within a unit, its shared partitions
  // (S < 0: the unit's first item, S from the scan)
  auto plan_item = [&](int unit, int p, Plan& pl, int m = 0, int S = -1) {
    if (unit < total) {
      const int j = unit / a.hkv;
      pl.it.unit = unit;
      pl.it.g = unit - j * a.hkv;
      pl.it.p = p;
      pl.it.tok0 = p * kPartition;
      if constexpr (SH) {
        const uint32_t v = static_cast<uint32_t>(sc.order[j]);
        pl.it.b0 = static_cast<int>(v & 2047u);
        pl.it.ucnt = static_cast<int>((v >> 11) & 15u) + 1;
        pl.it.S = S >= 0 ? S : static_cast<int>(v >> 16);
        pl.it.m = m;
        pl.it.stacked = p < pl.it.S ? 1 : 0;
      }
      if (SH && pl.it.stacked) {
        pl.it.b = pl.it.b0;
        pl.it.np = 0;
        pl.it.tok1 = pl.it.tok0 + kPartition;
      } else {
        pl.it.b = SH ? pl.it.b0 + m : sc.order[j];
        const int n = sc.n[pl.it.b];
        pl.it.np = partitions_of(n);
        pl.it.tok1 = min(n, pl.it.tok0 + kPartition);
      }
    } else {
      pl.it = QItem{unit, 0, 0, 0, 1, 0, 0, 0, 1, 0, 0, 0};
    }
    make_uniform(pl.it);
    if constexpr (SH) make_uniform_stack(pl.it);
    if constexpr (FUSED) {
      pl.pn = (pl.it.unit < total && pl.it.p == pl.it.np - 1 && pl.it.tok1 > pl.it.tok0)
                  ? pl.it.tok1 - 1
                  : -1;
      const int64_t row = (static_cast<int64_t>(pl.it.b) * a.hkv + pl.it.g) * D;
      const auto kr = tile_rsrc(static_cast<const uint16_t*>(a.k_new) + row, pl.pn >= 0 ? D * 2 : 0);
      const auto vr = tile_rsrc(static_cast<const uint16_t*>(a.v_new) + row, pl.pn >= 0 ? D * 2 : 0);
      pl.knew = __builtin_amdgcn_raw_buffer_load_b128(kr, (lane & (D / 8 - 1)) * 16, 0, kCached);
      pl.vnew = __builtin_amdgcn_raw_buffer_load_b32(vr, lane * 4, 0, kCached);  // D 64: lanes < 32
    }
    const int32_t* trow = a.tables + static_cast<int64_t>(pl.it.b) * a.mb;
    const int l = lane < 2 * kSteps ? lane : 0;
    const int base =
        (pl.it.tok0 + kStep * (wave + kWaves * (l >> 1))) / BS + (BS == 16 ? (l & 1) : 0);
    pl.ent = trow[min(base, a.mb - 1)];
    if constexpr (SH) {
      if (pl.it.stacked) {
        // the same 16 entries of every member (16 lanes per member)
        const int lm = lane & (2 * kSteps - 1);
        const int bm =
            (pl.it.tok0 + kStep * (wave + kWaves * (lm >> 1))) / BS + (BS == 16 ? (lm & 1) : 0);
#pragma unroll
        for (int k = 0; k < kStackRows / 4; ++k) {
          const int mm = min(4 * k + (lane >> 4), pl.it.ucnt - 1);
          pl.entm[k] = 4 * k < pl.it.ucnt
                           ? a.tables[static_cast<int64_t>(pl.it.b0 + mm) * a.mb + min(bm, a.mb - 1)]
                           : 0;
        }
      }
    }
  };
  // Query rows g*G .. g*G+G-1 of an item, loaded right before the item's first
  // KV loads, so that waiting for those covers these. Lanes past the group
  // repeat row G-1: those padding rows are never stored, and they are fully
  // masked wherever a step reaches past the context.
  auto load_query = [&](const Plan& pl, bf16x8 (&qv)[KS]) {
    // a stacked item's column r is head r % G of member r / G
    const int rr = min(r, rows_of(pl.it) - 1);
    const int bq = (SH && pl.it.stacked) ? pl.it.b0 + rr / G : pl.it.b;
    const int hh = (SH && pl.it.stacked) ? rr % G : rr;
    const uint16_t* qr =
        q + (static_cast<int64_t>(bq) * a.hq + pl.it.g * G + hh) * D + 8 * kg;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) qv[s2] = __builtin_bit_cast(bf16x8, ld16(qr + 32 * s2));
  };
  auto block_ids = [&](Plan& pl) {
#pragma unroll
    for (int s2 = 0; s2 < kSteps; ++s2) {
      const int t0 = pl.it.tok0 + kStep * (wave + kWaves * s2);
      const bool valid = t0 < pl.it.tok1;
      const int ia = __builtin_amdgcn_readlane(pl.ent, 2 * s2);
      const int ib = __builtin_amdgcn_readlane(pl.ent, 2 * s2 + 1);  // bs 32: unused
      pl.idA[s2] = valid ? clamp_block(ia, a.nb) : 0;
      pl.idB[s2] = (valid && BS == 16 && t0 + 16 < pl.it.tok1) ? clamp_block(ib, a.nb)
                                                                : pl.idA[s2];
    }
    if constexpr (SH) {
      bool same = true;
      if (pl.it.stacked) {
        const int lead = __shfl(pl.ent, lane & (2 * kSteps - 1));
#pragma unroll
        for (int k = 0; k < kStackRows / 4; ++k)
          if (4 * k < pl.it.ucnt) same = same && pl.entm[k] == lead;
      }
      pl.ok = __builtin_amdgcn_ballot_w64(!same) == 0;
    }
  };
  // SH: a shared item whose block ids are not every member's (some wave saw
  // a difference) becomes b0's own item of the same partition, and the unit's
  // later items run unstacked: S drops to this partition. Its loads (b0's
  // blocks) are already the right ones, and its query columns 0 .. G-1 are
  // b0's heads either way.
  auto unstack_unless_ok = [&](Plan& pl, const int (&ok)[kWaves]) {
    if constexpr (SH) {
      if (pl.it.stacked && !(ok[0] && ok[1] && ok[2] && ok[3])) {
        static_assert(kWaves == 4, "one flag per wave");
        pl.it.S = pl.it.p;
        pl.it.stacked = 0;
        pl.it.m = 0;
        const int n = sc.n[pl.it.b0];
        pl.it.np = partitions_of(n);
        pl.it.tok1 = min(n, pl.it.tok0 + kPartition);
        make_uniform(pl.it);
        make_uniform_stack(pl.it);
      }
    }
  };
  Eng eng;
  typename Eng::KV kv[2];
  auto issue_ids = [&](int g, int idA, int idB, bool live, typename Eng::KV& buf) {
    const int64_t kofs = static_cast<int64_t>(g) * BS * D;
    const int64_t vofs = static_cast<int64_t>(a.hkv) * BS * D + static_cast<int64_t>(g) * D * BS;
    eng.template load_kv<POL>(buf, pool, a.blk_elems, kofs, vofs, idA, idB, lane, live);
  };
  auto issue = [&](const Plan& pl, int s2, typename Eng::KV& buf) {
    issue_ids(pl.it.g, pl.idA[s2], pl.idB[s2],
              pl.it.tok0 + kStep * (wave + kWaves * s2) < pl.it.tok1, buf);
  };
  // FUSED: in the step starting at t0 that holds the new token, its K (the
  // lanes of its token row r, set a or b) and its V (the lanes of its 4-token
  // slice, one 16-bit half of one word) become the token's own.
  auto patch = [&](typename Eng::KV& kv, int t0, const Plan& pl) {
    if constexpr (FUSED) {
      if (t0 <= pl.pn && pl.pn < t0 + kStep) {  // wave-uniform
        const int tl = pl.pn - t0, t16 = tl & 15;
        const bool setb = tl >= 16;
        // (each field written unconditionally: one store through a pointer
        // chosen between kA and kB would keep the step in scratch memory too)
        const bool ka = r == t16 && !setb, kb = r == t16 && setb;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          u32x4 k;  // slice kg + 4 s2
#pragma unroll
          for (int x = 0; x < 4; ++x) k[x] = __shfl(pl.knew[x], kg + 4 * s2);
          kv.kA[s2] = ka ? k : kv.kA[s2];
          kv.kB[s2] = kb ? k : kv.kB[s2];
        }
        // word w = 2 (set b) + (t16 % 4) / 2 of the lanes of slice t16 / 4,
        // 16-bit half t16 % 2; the per-word masks are plain arithmetic, so
        // that no word is picked by a run-time index (which would move the
        // step's registers to scratch memory)
        const int w = (setb ? 2 : 0) + ((t16 & 3) >> 1);
        const int sh = 16 * (t16 & 1);
        const uint32_t sel = kg == (t16 >> 2) ? 1u << w : 0u;
        uint32_t msk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) msk[e] = (0u - ((sel >> e) & 1u)) & (0xFFFFu << sh);
#pragma unroll
        for (int j = 0; j < Eng::VT; ++j) {
          // dimension r + 16 j: half r % 2 of lane (r + 16 j) / 2's pair
          const uint32_t d2 = __shfl(pl.vnew, (r + 16 * j) >> 1);
          const uint32_t v = ((d2 >> (16 * (r & 1))) & 0xFFFFu) << sh;
#pragma unroll
          for (int e = 0; e < 4; ++e) kv.vv[j][e] = (kv.vv[j][e] & ~msk[e]) | (v & msk[e]);
        }
      }
    }
  };

  // The wave states of item i are combined and folded while item i+1's steps
  // are in flight (after its third and fourth steps' loads are issued), so
  // that this never stands between a step's arrival and the next loads.
  // Thread c < G*C4 owns output row c / C4, dimensions 4 (c % C4) .. +3, of
  // every unit: a sequence of one partition stores its normalised output
  // directly; otherwise each partition's normalised output, rounded to bf16
  // as a stored partial would be, is folded into the thread's merge state,
  // and the last partition stores the merged row.
  MergeState ms;
  ms.reset();
  // SH: partial p of row (sequence b, query head g*G + h) in the workspace, in
  // the split-K merge's layout: element offset of o (times D) and of (M, L)
  // (times 2)
  auto partial_at = [&](int b, int g, int h, int p) -> int64_t {
    return (static_cast<int64_t>(b) * a.hq + g * G) * a.np_max + static_cast<int64_t>(p) * G + h;
  };
  uint16_t* ws_o = static_cast<uint16_t*>(a.ws_o);
  auto publish = [&](const MergeSmem<D, R>& sm, const QItem& it) {
    const int c = threadIdx.x;
    if constexpr (SH) {
      if (it.stacked) {  // every member's partial of this shared partition
        const int rows = it.ucnt * G;
        for (int row = c / C4; row < rows; row += kWaves * 64 / C4) {
          const int dd = 4 * (c % C4);
          float M, L;
          f32x4 O;
          combine_waves(sm, row, dd, M, L, O);
          const float inv = L > 0.f ? 1.f / L : 0.f;
          const int mm = row / G, h = row - mm * G;
          const int64_t at = partial_at(it.b0 + mm, it.g, h, it.p);
          store4<uint16_t>(ws_o + at * D + dd, O * inv);
          if (dd == 0) {
            a.ws_ml[2 * at] = M;
            a.ws_ml[2 * at + 1] = L;
          }
        }
        return;
      }
    }
    if (c >= G * C4) return;
    const int row = c / C4, dd = 4 * (c - row * C4);
    float M, L;
    f32x4 O;
    combine_waves(sm, row, dd, M, L, O);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(a.out) +
                     (static_cast<int64_t>(it.b) * a.hq + it.g * G + row) * D + dd;
    if (it.np == 1) {
      store4<uint16_t>(orow, O * inv);
      return;
    }
    if (it.p == 0) ms.reset();
    if constexpr (SH) {
      if (it.p == it.S && it.S > 0) {
        // a stacked member's first own partition: its shared partitions'
        // partials first, as stored, in partition order (other waves of this
        // workgroup stored them while an earlier item ran; that item's closing
        // __syncthreads, a workgroup-scope release and acquire, orders those
        // stores before these loads)
        ms.reset();
        for (int p2 = 0; p2 < it.S; ++p2) {
          const int64_t at = partial_at(it.b, it.g, row, p2);
          ms.fold(a.ws_ml[2 * at], a.ws_ml[2 * at + 1], load4<uint16_t>(ws_o + at * D + dd));
        }
      }
    }
    ms.fold(M, L, as_stored<uint16_t>(O * inv));
    if (it.p == it.np - 1) store4<uint16_t>(orow, ms.result());
  };

  if (rank < 0) {
    if (threadIdx.x == 0) {
      s_next[0] = 2 * dealt + atomicAdd(&queue[0], 1);
      s_next[1] = 2 * dealt + atomicAdd(&queue[0], 1);
    }
    __syncthreads();
  }
  int cur_u = rank < 0 ? s_next[0] : rank;
  int ahead_u = rank < 0 ? s_next[1] : 2 * dealt - 1 - rank;
  __syncthreads();  // both slots read before either is rewritten
  int parity = 0;
  Plan cur, nxt;
  QItem prev;  // the item whose states wait in sm2[parity ^ 1]
  bool have_prev = false;
  bf16x8 qcur[KS], qnxt[KS];
  plan_item(cur_u, 0, cur);
  block_ids(cur);
  if constexpr (SH) {  // the first item's check, before anything relies on it
    if (lane == 0) ds.s_ok[1][wave] = cur.ok ? 1 : 0;
    __syncthreads();
    unstack_unless_ok(cur, ds.s_ok[1]);
  }
  load_query(cur, qcur);
  issue(cur, 0, kv[0]);
  issue(cur, 1, kv[1]);
  while (cur.it.unit < total) {
    // the next item: the current unit's next partition, else the unit taken
    // ahead (and then another unit is taken from the queue during this item).
    // SH: a unit's shared partitions, then each member's own partitions.
    bool new_unit;
    if constexpr (SH) {
      const QItem& c = cur.it;
      if (c.stacked) {
        new_unit = false;
        plan_item(c.unit, c.p + 1 < c.S ? c.p + 1 : c.S, nxt, 0, c.S);
      } else if (c.p + 1 < c.np) {
        new_unit = false;
        plan_item(c.unit, c.p + 1, nxt, c.m, c.S);
      } else if (c.m + 1 < c.ucnt) {
        new_unit = false;
        plan_item(c.unit, c.S, nxt, c.m + 1, c.S);
      } else {
        new_unit = true;
        plan_item(ahead_u, 0, nxt);
      }
    } else {
      new_unit = cur.it.p + 1 >= cur.it.np;
      plan_item(new_unit ? ahead_u : cur.it.unit, new_unit ? 0 : cur.it.p + 1, nxt);
    }
    int after_id = 0;
    eng.init();
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) eng.qreg[0][s2] = qcur[s2];
    if (r < rows_of(cur.it)) eng.lim[0] = cur.it.tok1 - 1;
    // -- steps of the current item; the next item's first two steps follow ------
    if constexpr (!HANDOVER) {
#pragma unroll
    for (int s2 = 0; s2 < kSteps; ++s2) {
      const int t0 = cur.it.tok0 + kStep * (wave + kWaves * s2);
      if (t0 < cur.it.tok1) {
        patch(kv[s2 & 1], t0, cur);
        eng.compute(kv[s2 & 1], t0, cur.it.tok1, lane, a.sl2e);
      }
      if (s2 == kSteps - 2 && new_unit && threadIdx.x == 0) {
        // Take the unit after next; the id goes to LDS just before the
        // barrier, when waiting for it no longer holds back any load.
        after_id = 2 * dealt + atomicAdd(&queue[0], 1);
      }
      if (s2 == kSteps - 2) {
        block_ids(nxt);
        load_query(nxt, qnxt);
      }
      if (s2 + 2 < kSteps)
        issue(cur, s2 + 2, kv[s2 & 1]);
      else
        issue(nxt, s2 + 2 - kSteps, kv[s2 & 1]);
      if (s2 == 1 && have_prev) publish(sm2[parity ^ 1], prev);
    }
    } else {
    // This wave's steps of the item: `live` of them reach into it; they are
    // taken in pairs (kv[0], kv[1]), lw in all. As soon as the last pair's
    // buffers free up, the next item's steps 0 and 1 are issued into them, so
    // a short item hands over to the next one at once instead of first
    // running out its dead steps. The pairs nest, so every load on a path is
    // issued unconditionally and the compiler's wait counts stay exact.
    static_assert(kSteps == 8, "four pairs of steps per wave and item");
    const int len = cur.it.tok1 - cur.it.tok0;
    const int live = len > kStep * wave ? (len - kStep * wave + kWaves * kStep - 1) / (kWaves * kStep)
                                        : 0;
    const int lw = min(kSteps, (live + 1) & ~1);
    // The hand-over: take the unit after next (the id goes to LDS just before
    // the barrier, when waiting for it no longer holds back any load), the
    // next item's block ids and its query rows (read when it starts, by which
    // time every load issued before them has been waited for anyway).
    auto hand_over = [&]() {
      if (new_unit && threadIdx.x == 0) after_id = 2 * dealt + atomicAdd(&queue[0], 1);
      block_ids(nxt);
      load_query(nxt, qnxt);
    };
    // step s (static) of the current item into / out of kv[s & 1], then the
    // load of step s + 2, or of the next item's step s & 1 after the last pair
    auto step_and_issue = [&](auto sc, bool last) {
      constexpr int s = decltype(sc)::value;
      const int t0 = cur.it.tok0 + kStep * (wave + kWaves * s);
      if (t0 < cur.it.tok1) {
        patch(kv[s & 1], t0, cur);
        eng.compute(kv[s & 1], t0, cur.it.tok1, lane, a.sl2e);
      }
      if ((s & 1) == 0 && last) hand_over();
      const int idA = last ? nxt.idA[s & 1] : (s + 2 < kSteps ? cur.idA[(s + 2) % kSteps] : 0);
      const int idB = last ? nxt.idB[s & 1] : (s + 2 < kSteps ? cur.idB[(s + 2) % kSteps] : 0);
      const int g = last ? nxt.it.g : cur.it.g;
      const bool lv = last ? nxt.it.tok0 + kStep * (wave + kWaves * (s & 1)) < nxt.it.tok1
                           : cur.it.tok0 + kStep * (wave + kWaves * (s + 2)) < cur.it.tok1;
      issue_ids(g, idA, idB, lv, kv[s & 1]);
    };
    auto pair = [&](auto pc, bool last) {
      constexpr int s = decltype(pc)::value;
      step_and_issue(std::integral_constant<int, s>{}, last);
      step_and_issue(std::integral_constant<int, s + 1>{}, last);
      if (s == 0 && have_prev) publish(sm2[parity ^ 1], prev);
    };
    if (lw == 0) {  // nothing of this item for this wave
      hand_over();
      issue_ids(nxt.it.g, nxt.idA[0], nxt.idB[0], nxt.it.tok0 + kStep * wave < nxt.it.tok1, kv[0]);
      issue_ids(nxt.it.g, nxt.idA[1], nxt.idB[1],
                nxt.it.tok0 + kStep * (wave + kWaves) < nxt.it.tok1, kv[1]);
      if (have_prev) publish(sm2[parity ^ 1], prev);
    } else {
      pair(std::integral_constant<int, 0>{}, lw == 2);
      if (lw > 2) {
        pair(std::integral_constant<int, 2>{}, lw == 4);
        if (lw > 4) {
          pair(std::integral_constant<int, 4>{}, lw == 6);
          if (lw > 6) pair(std::integral_constant<int, 6>{}, true);
        }
      }
    }
    }
    // -- leave the wave states of the current item ---------------------------------
    // One barrier per item: the wave states and the queue slot alternate
    // between two LDS copies. Item i's copy is read (folded) during item i+1
    // and rewritten by item i+2, after item i+1's barrier.
    if (threadIdx.x == 0 && new_unit) s_next[parity] = after_id;
    if constexpr (SH) {
      if (lane == 0) ds.s_ok[parity][wave] = nxt.ok ? 1 : 0;
    }
    MergeSmem<D, R>& sm = sm2[parity];
    const float lt = sum_over_groups(eng.l[0]);
    if (r < rows_of(cur.it)) {
      if (kg == 0) {
        sm.m[wave][r] = eng.m[0];
        sm.l[wave][r] = lt;
      }
#pragma unroll
      for (int j = 0; j < D / 16; ++j)
        *reinterpret_cast<f32x4*>(&sm.o[wave][r][16 * j + 4 * kg]) = eng.o[0][j];
    }
    __syncthreads();
    if (new_unit) ahead_u = s_next[parity];
    unstack_unless_ok(nxt, ds.s_ok[parity]);
    prev = cur.it;
    have_prev = true;
    parity ^= 1;
    cur = nxt;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) qcur[s2] = qnxt[s2];
  }
  if (have_prev) publish(sm2[parity ^ 1], prev);
}

// The whole decode of one workgroup: scan, then the loop under the call's
// cache policy (the same in every workgroup: it depends only on the inputs).
// rank, dealt: see decode_loop.
template <int D, int BS, bool SH = false, int R = kMaxGroup, bool HANDOVER = false,
          bool FUSED = false>
__device__ __forceinline__ void decode_persistent(const DecodeArgs& a, int32_t* __restrict__ queue,
                                                  DecodeSmem<D, R>& ds, int rank, int dealt) {
  // The hand-over pays where loads return quickly and items are short
  // (cached calls: shared prefixes, small batches). A streaming call keeps
  // every wave's loads back to back instead: there the hand-over's extra
  // branches make the loads wait more (measured 226 -> 237 us on the GQA
  // long-tail batch), while it gains 124 -> 106 us on the shared-prefix batch.
  if (decode_scan<D, BS, SH>(a, queue, ds))
    decode_loop<D, BS, kCached, SH, R, HANDOVER, FUSED>(a, queue, ds, rank, dealt);
  else
    decode_loop<D, BS, kNontemporal, SH, R, false, FUSED>(a, queue, ds, rank, dealt);
}

// (launched one workgroup per compute unit: see launch_decode_bf16)
template <int D, int BS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_bf16_persistent_kernel(DecodeArgs a, int32_t* __restrict__ queue) {
  __shared__ DecodeSmem<D> ds;
  decode_persistent<D, BS, false, kMaxGroup, true>(a, queue, ds, blockIdx.x, gridDim.x);
  leave_queue(queue);
}

// The same with the caller's sharing hint: stacked units, whose wave states
// take kStackRows rows (more LDS than two workgroups per compute unit leave,
// so one per unit, as the launch uses anyway).
template <int D, int BS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_bf16_shared_kernel(DecodeArgs a, int32_t* __restrict__ queue) {
  __shared__ DecodeSmem<D, kStackRows> ds;
  decode_persistent<D, BS, true, kStackRows, true>(a, queue, ds, blockIdx.x, gridDim.x);
  leave_queue(queue);
}

// The append of a fused decode step: every (sequence, kv head)'s new token
// goes to its slot. No read of this call needs the slot's contents (the wave
// whose step holds the position uses k_new / v_new instead, and a slot being
// appended to belongs to its sequence alone), so the stores may land at any
// time. Workgroup w takes pairs w, w + W, ... (W workgroups), wave v of them
// every fourth. The first kAppendRound pairs of each wave are loaded before
// the scan, in its round trip, and stored after the loop, when no wait of the
// wave's loads can be held back by them (stored right after the scan instead,
// they made the step 4.6% slower); any further pairs (over kAppendRound * 4 * W
// of them) are loaded and stored after the loop.
constexpr int kAppendRound = 2;
template <int D>
struct AppendRound {
  u32x4 k[kAppendRound];     // lane < D/8: K slice `lane`
  uint32_t v[kAppendRound];  // V dimensions 2 lane, 2 lane + 1 (D 64: lanes < 32)
  int slot[kAppendRound];    // wave-uniform; -1: nothing to write
  int pr[kAppendRound];
};
template <int D, int BS>
__device__ __forceinline__ void append_load(const DecodeArgs& a, AppendRound<D>& ar, int first) {
  const int pairs = a.num_seqs * a.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int stride = static_cast<int>(gridDim.x) * kWaves;
#pragma unroll
  for (int k = 0; k < kAppendRound; ++k) {
    const int pr = first + (static_cast<int>(blockIdx.x) * kWaves + wave) + k * stride;
    const bool in = pr < pairs;
    const int b = in ? pr / a.hkv : 0;
    const int64_t src = (static_cast<int64_t>(in ? pr : 0)) * D;
    const auto kr = tile_rsrc(static_cast<const uint16_t*>(a.k_new) + src, in ? D * 2 : 0);
    const auto vr = tile_rsrc(static_cast<const uint16_t*>(a.v_new) + src, in ? D * 2 : 0);
    ar.k[k] = __builtin_amdgcn_raw_buffer_load_b128(kr, (lane & (D / 8 - 1)) * 16, 0, kCached);
    ar.v[k] = __builtin_amdgcn_raw_buffer_load_b32(vr, lane * 4, 0, kCached);
    ar.slot[k] = in ? a.slots[b] : -1;
    ar.pr[k] = pr;
  }
}
template <int D, int BS>
__device__ __forceinline__ void append_store(const DecodeArgs& a, const AppendRound<D>& ar) {
  const int lane = threadIdx.x & 63;
  uint16_t* pool = static_cast<uint16_t*>(const_cast<void*>(a.pool));
#pragma unroll
  for (int k = 0; k < kAppendRound; ++k) {
    const int slot = __builtin_amdgcn_readfirstlane(ar.slot[k]);
    if (slot < 0 || static_cast<int64_t>(slot) >= a.nb * BS) continue;  // wave-uniform
    const int g = ar.pr[k] - (ar.pr[k] / a.hkv) * a.hkv;
    const int64_t blk = slot / BS;
    const int off = slot - static_cast<int>(blk) * BS;
    uint16_t* base = pool + blk * a.blk_elems;
    // K: lane < D/8 writes 8-element slice `lane` at the slot
    if (lane < D / 8)
      st16(base + static_cast<int64_t>(g) * BS * D + (static_cast<int64_t>(lane) * BS + off) * 8,
           ar.k[k]);
    // V: dimension d sits at element (off/4 * D + d) * 4 + off%4 of the tile
    uint16_t* vt = base + static_cast<int64_t>(a.hkv) * BS * D + static_cast<int64_t>(g) * D * BS;
    if (2 * lane < D) {
      const int64_t e = ((off >> 2) * D + 2 * lane) * 4 + (off & 3);
      vt[e] = static_cast<uint16_t>(ar.v[k]);
      vt[e + 4] = static_cast<uint16_t>(ar.v[k] >> 16);
    }
  }
}

// pa_decode of a decode step together with its append (one launch: see
// decode_loop's FUSED, append_load and append_store).
template <int D, int BS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_bf16_append_kernel(DecodeArgs a, int32_t* __restrict__ queue) {
  __shared__ DecodeSmem<D> ds;
  AppendRound<D> ar;
  append_load<D, BS>(a, ar, 0);
  const bool cached = decode_scan<D, BS, false>(a, queue, ds);
  if (cached)
    decode_loop<D, BS, kCached, false, kMaxGroup, true, true>(a, queue, ds, blockIdx.x, gridDim.x);
  else
    decode_loop<D, BS, kNontemporal, false, kMaxGroup, false, true>(a, queue, ds, blockIdx.x,
                                                                    gridDim.x);
  append_store<D, BS>(a, ar);
  // pairs past the first round (batches of more than kAppendRound * 4 * W)
  const int round = static_cast<int>(gridDim.x) * kWaves * kAppendRound;
  for (int first = round; first < a.num_seqs * a.hkv; first += round) {
    append_load<D, BS>(a, ar, first);
    append_store<D, BS>(a, ar);
  }
  leave_queue(queue);
}

template <int D, int BS, int G>
__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeArgs a) {
  DecodeItem it;
  if (!decode_item<BS>(a, it)) return;
  __shared__ MergeSmem<D> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, c = lane & 15;
  const float* pool = static_cast<const float*>(a.pool);
  const float* q = static_cast<const float*>(a.q);
  const int64_t row0 = static_cast<int64_t>(it.b) * a.hq + it.g * G;

  F32Engine<D, BS, G> eng;
  eng.init(q + row0 * D, c);
  eng.lim = it.tok1 - 1;
  const int64_t kofs = static_cast<int64_t>(it.g) * BS * D;
  const int64_t vofs = static_cast<int64_t>(a.hkv) * BS * D + static_cast<int64_t>(it.g) * D * BS;
  const int32_t* trow = a.tables + static_cast<int64_t>(it.b) * a.mb;
  for (int t0 = it.tok0 + wave * kStep; t0 < it.tok1; t0 += kWaves * kStep) {
    int blkA, blkB;
    step_blocks<BS>(trow, t0, it.tok1, a.nb, blkA, blkB);
    eng.step(pool, a.blk_elems, kofs, vofs, blkA, blkB, t0, it.tok1, lane, a.sl2e);
  }
#pragma unroll
  for (int qi = 0; qi < G; ++qi) {
    const float lt = sum_over_groups(eng.l[qi]);
#pragma unroll
    for (int k = 0; k < F32Engine<D, BS, G>::EPL; ++k) {
      const float v = sum_over_groups(eng.acc[qi][k]);
      if (grp == 0) sm.o[wave][qi][c + 16 * k] = v;
    }
    if (lane == 0) {
      sm.m[wave][qi] = eng.m[qi];
      sm.l[wave][qi] = lt;
    }
  }
  __syncthreads();
  finish_partition<D, float>(sm, G, it.np, it.p, static_cast<float*>(a.out) + row0 * D,
                             static_cast<float*>(a.ws_o) + row0 * a.np_max * D,
                             a.ws_ml + row0 * a.np_max * 2);
}

// Split-K merge: one workgroup per (sequence, kv head) with more than one
// partition combines the partitions' (M, L, o = O / L) by the log-sum-exp
// identity M* = max M_j, L* = sum L_j 2^(M_j - M*),
// out = sum L_j 2^(M_j - M*) o_j / L*.
template <int D, int BS, typename OutT>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  // One workgroup per (sequence, kv head) with more than one partition; each
  // thread combines four output dimensions of one row. It reads the (M, L)
  // of its row itself (the 32 or 16 threads of a row read the same words), so
  // there is no barrier: the partials are read in batches of kBatch
  // partitions, all loads of a batch issued together, and folded one by one
  // (MergeState).
  constexpr int C4 = D / 4;
  constexpr int kBatch = 8;
  const int bg = blockIdx.x;
  if (bg >= a.num_seqs * a.hkv) return;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  int n = a.lens[b];
  n = n < 0 ? 0 : n;
  n = n > a.max_ctx ? a.max_ctx : n;
  n = n > a.mb * BS ? a.mb * BS : n;
  const int np = (n + kPartition - 1) / kPartition;
  if (np <= 1) return;
  const int G = a.hq / a.hkv;
  const int row = threadIdx.x / C4, c4 = threadIdx.x - row * C4;
  if (row >= G) return;
  const int64_t row0 = static_cast<int64_t>(b) * a.hq + g * G;
  // partition pp of this row: (M, L) at mlr[2 * G * pp], o at orow[pp * G * D]
  const float* mlr = a.ws_ml + row0 * a.np_max * 2 + 2 * row;
  const OutT* orow = static_cast<const OutT*>(a.ws_o) + row0 * a.np_max * D + row * D + 4 * c4;
  MergeState st;
  st.reset();
  for (int p0 = 0; p0 < np; p0 += kBatch) {
    float2 ml[kBatch];
    f32x4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {  // past the last partition: re-read it, unused
      const int pp = min(p0 + u, np - 1);
      ml[u] = *reinterpret_cast<const float2*>(mlr + 2 * G * pp);
      v[u] = load4<OutT>(orow + static_cast<int64_t>(pp) * G * D);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (p0 + u < np) st.fold(ml[u].x, ml[u].y, v[u]);
  }
  store4<OutT>(static_cast<OutT*>(a.out) + (row0 + row) * D + 4 * c4, st.result());
}

// ---------------------------------------------------------------------------
// Prefill MFMA engine: online-softmax attention of one tile of 32 query rows
// over 32-token steps, on v_mfma_f32_32x32x16_bf16. That form runs at the
// matrix cores' full rate on this target, takes half the instructions of the
// 16x16 form for the same work (each MFMA instruction also costs the VALU a
// few issue cycles), and gives each lane 16 scores of one row, so a row's
// maximum needs a single lane swap.
//
// Lane (h = lane/32, j = lane%32); "quad" c of a step = its tokens 4c..4c+3.
//   score MFMA s (dims 16s .. 16s+15)   S^T[tok][row] = K[tok][:] . Q[row][:]
//     A (K)   lane gives token j, dims 16s + 8h .. +7 (one 8-element K slice)
//     B (Q)   lane gives row j at the same dims
//     C       lane holds row j at token 8p + 4h + i as element 4p + i (p, i < 4),
//             that is quads h, 2+h, 4+h, 6+h
//   p.V MFMA (dim block db, half m)     O^T[dim][row] += V^T[dim][tok] . P^T[tok][row]
//     B (P)   lane gives row j at quads 4m+h and 4m+2+h: elements 8m .. 8m+7 of
//             its own scores, so probabilities never leave registers
//     A (V^T) lane gives dim 32db + j at the same eight tokens
//     C       lane holds O^T[32db + 8p + 4h + i][j] as element 4p + i
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int D>
struct PrefillEngine {
  static constexpr int KS = D / 16;  // score MFMAs (and K operands) per step
  static constexpr int DB = D / 32;  // 32-dim blocks of O^T
  bf16x8 qreg[KS];
  f32x16 o[DB];
  float m, l;
  int lim;  // last token this lane's row may attend to (-1: none)

  __device__ __forceinline__ void init() {
    m = kNoMax;
    l = 0.f;
    lim = -1;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) qreg[s] = bf16x8{};
  }

  __device__ __forceinline__ void load_q(const uint16_t* q_row, int h) {
#pragma unroll
    for (int s = 0; s < KS; ++s) qreg[s] = __builtin_bit_cast(bf16x8, ld16(q_row + 16 * s + 8 * h));
  }

  __device__ __forceinline__ f32x16 scores(const u32x4 (&k)[KS]) const {
    f32x16 sc = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k[s]), qreg[s], sc, 0,
                                                   0, 0);
    return sc;
  }

  // Tokens >= vend get their V zeroed (they may be NaN) and scores of tokens
  // past the row's limit become -inf, where the step reaches that far.
  // vv[2 * db + m] is the V^T operand of dim block db, half m.
  __device__ __forceinline__ void edge_masks(f32x16& sc, u32x4 (&vv)[2 * DB], int t0, int vend,
                                             int h) const {
    if (t0 + 32 > vend) {  // wave-uniform
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // word w holds elements 2w, 2w+1: quad 4mh + h (w < 2) or 4mh + 2 + h
          const int quad = 4 * mh + h + 2 * (w >> 1);
          const int n = vend - (t0 + 4 * quad);
          const int e0 = 2 * (w & 1);
          const uint32_t mask = (e0 < n ? 0x0000FFFFu : 0u) | (e0 + 1 < n ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int db = 0; db < DB; ++db) vv[2 * db + mh][w] &= mask;
        }
      }
    }
    // Only steps that reach past the limit of some real row need the score
    // mask; then padding rows (lim < 0) are masked entirely, otherwise their
    // scores are finite and never read.
    if (__builtin_amdgcn_ballot_w64(lim >= 0 && t0 + 31 > lim) != 0) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[4 * p + i] = (t0 + 8 * p + 4 * h + i <= lim) ? sc[4 * p + i] : -__builtin_inff();
    }
  }

  // bf16 weights exp2(s * sl2e - mref) of this lane's 16 scores, and their sum
  // (two chains of four bf16 pair sums).
  __device__ __forceinline__ float weights(const f32x16& sc, float sl2e, float mref,
                                           bf16x8 (&p)[2]) const {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      p[e >> 3][e & 7] = static_cast<__bf16>(exp2_fast(fmaf(sc[e], sl2e, -mref)));
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
      ps[mh] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p[mh], p[mh], 0, 1), kOnes2, ps[mh], false);
      ps[mh] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p[mh], p[mh], 2, 3), kOnes2, ps[mh], false);
      ps[mh] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p[mh], p[mh], 4, 5), kOnes2, ps[mh], false);
      ps[mh] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p[mh], p[mh], 6, 7), kOnes2, ps[mh], false);
    }
    return ps[0] + ps[1];
  }

  // Online softmax and p.V on scores already masked (see Bf16Engine for the
  // rescale slack and the bf16 weight sums). The weights are first taken
  // against the row's reference maximum m. Every weight is non-negative and at
  // most its lane's sum, so while every lane's sum stays below 2^kRescaleSlack
  // no score has passed m + kRescaleSlack, the state needs no rescale, and the
  // row's maximum is not needed at all. Otherwise (a row's first keys, whose m
  // is kNoMax, make the sums infinite; so does a NaN) the wave takes the
  // maximum and applies the rescale rule, recomputing the weights of the rows
  // whose reference moves.
  __device__ __forceinline__ void softmax_pv(const f32x16& sc, const u32x4 (&vv)[2 * DB],
                                             float sl2e) {
    bf16x8 p[2];
    float ps = weights(sc, sl2e, m, p);
    if (__builtin_amdgcn_ballot_w64(!(ps < kSlackWeight)) != 0) {  // wave-uniform
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = smax(mx, sc[e]);
      {  // the other half of the row (lane ^ 32)
        const uint32_t u = __float_as_uint(mx);
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        mx = smax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float mtop = smax(m, mx * sl2e);
      const bool grow = mtop > m + kRescaleSlack;
      const float mnew = grow ? mtop : m;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        ps = weights(sc, sl2e, mnew, p);  // rows that keep m get the same weights
        if (__builtin_amdgcn_ballot_w64(grow && m != kNoMax) != 0) {
          const float alpha = exp2_fast(m - mnew);
          l *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db] *= alpha;
        }
      }
      m = mnew;
    }
    l += ps;
#pragma unroll
    for (int mh = 0; mh < 2; ++mh)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv[2 * db + mh]),
                                                        p[mh], o[db], 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Chunked prefill.
// ---------------------------------------------------------------------------
struct PrefillArgs {
  void* out;
  const void* q;
  const void* pool;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* qsl;
  int num_chunks, total_q, mb, hq, hkv;
  int64_t nb, blk_elems;
  float sl2e;
};

// Chunk geometry: queries q0 .. q0+L-1 at positions prior .. prior+L-1.
__device__ __forceinline__ bool chunk_geometry(const PrefillArgs& a, int c, int max_tokens, int& q0,
                                               int& L, int& prior) {
  q0 = a.qsl[c];
  L = a.qsl[c + 1] - q0;
  int n = a.lens[c];
  n = n > max_tokens ? max_tokens : n;
  if (q0 < 0 || L <= 0 || q0 + L > a.total_q || n < L) return false;
  prior = n - L;
  return true;
}

// bf16: a wave owns one tile of kPrefillRows rows; row R -> (position R / G,
// head R % G). The workgroup's four waves cover consecutive positions and
// share one key range, so each 32-token step of K and V is loaded from HBM
// once per workgroup (16-byte loads by all 256 threads, issued a step ahead)
// into one of two LDS buffers, and every wave reads its MFMA operands from
// there.
constexpr int kPrefillRows = 32;

template <int D>
struct PrefillSmem {
  uint16_t k[2][(D / 8) * kStep * 8];  // [slice][token][8], tokens of one step
  // [quad pair c][dim][8]: quad pair c = 2m + h holds quads 4m+h (elements
  // 0..3) and 4m+2+h (4..7), which is one lane's whole p.V operand for that
  // dim (PrefillEngine)
  uint16_t v[2][(kStep / 8) * D * 8];
};

// Waves of a prefill workgroup (W): at d 128 eight (two per SIMD, 256 rows
// sharing each step's K and V), at d 64 four (a step's 512 pieces are then
// one K and one V piece per thread).
constexpr int prefill_waves(int D) { return D == 128 ? 8 : kWaves; }

// One workgroup tile: positions x*W*pos_per_wave .. of chunk c, kv head g.
// Every branch that returns early is uniform over the workgroup, and every
// path that reaches the step loop runs the same barriers in every wave.
template <int D, int BS, int W>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, PrefillSmem<D>& smem, int x,
                                             int c, int g) {
  using Eng = PrefillEngine<D>;
  constexpr int KS = Eng::KS, DB = Eng::DB;
  constexpr int kThreads = 64 * W;
  constexpr int kChunks = 2 * D * kStep * 2 / 16;  // 16-byte pieces of one step's K and V
  constexpr int kPer = kChunks / kThreads;         // per thread
  static_assert(kChunks % kThreads == 0, "a step is a whole number of 16-byte pieces per thread");
  int q0, L, prior;
  if (!chunk_geometry(a, c, a.mb * BS, q0, L, prior)) return;  // uniform per workgroup
  const int G = a.hq / a.hkv;
  const int pos_per_wave = kPrefillRows / G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wg_i0 = x * W * pos_per_wave;
  if (wg_i0 >= L) return;  // uniform per workgroup
  const int i0 = wg_i0 + wave * pos_per_wave;
  const int r = lane & 31, h = lane >> 5;
  const uint16_t* pool = static_cast<const uint16_t*>(a.pool);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  // the two LDS buffers, through pointers that alias nothing else
  constexpr int kK = (D / 8) * kStep * 8, kV = (kStep / 8) * D * 8;
  uint16_t* __restrict__ lk = &smem.k[0][0];
  uint16_t* __restrict__ lv = &smem.v[0][0];

  Eng eng;
  eng.init();
  // this lane's row: position i, head hd
  const int i = i0 + r / G, hd = r - (r / G) * G;
  if (i < L) {
    eng.load_q(q + ((static_cast<int64_t>(q0) + i) * a.hq + g * G + hd) * D, h);
    eng.lim = prior + i;
  }
  // keys 0 .. kend-1 for this wave's rows, kend_wg for the workgroup's
  const int kend = prior + min(L, i0 + pos_per_wave);
  const int kend_wg = prior + min(L, wg_i0 + W * pos_per_wave);
  const int32_t* trow = a.tables + static_cast<int64_t>(c) * a.mb;
  const int64_t kofs = static_cast<int64_t>(g) * BS * D;
  const int64_t vofs = static_cast<int64_t>(a.hkv) * BS * D + static_cast<int64_t>(g) * D * BS;

  // Piece p of a step: K pieces first ([slice c][token t], one token's 8
  // dims), then V pieces: 2 dims x 4 tokens of one quad (the pool's V layout
  // is [quad][dim][4]). V piece 2m + w is dim pair m % (D/2) of quad pair
  // cp = m / (D/2), quad 4(cp/2) + cp%2 + 2w of the step. Adjacent lanes thus
  // hold the two quads of the same two dims, which the stash turns into two
  // whole LDS rows.
  // Returns the element offset inside the step's block (A: tokens 0..15 or,
  // at bs 32, all 32) and whether it comes from block B (bs 16, tokens 16..31).
  auto piece_src = [&](int u, int pc, bool& from_b) -> int64_t {
    if (u < kPer / 2) {
      const int sl = pc / kStep, t = pc - sl * kStep;
      from_b = BS == 16 && t >= 16;
      const int slot = BS == 16 ? (t & 15) : t;
      return kofs + (static_cast<int64_t>(sl) * BS + slot) * 8;
    }
    const int pv = pc - kChunks / 2;
    const int m = pv >> 1;
    const int cp = m / (D / 2), dp = m - cp * (D / 2);
    const int quad = 4 * (cp >> 1) + (cp & 1) + 2 * (pv & 1);
    from_b = BS == 16 && quad >= 4;
    const int bq = BS == 16 ? (quad & 3) : quad;
    return vofs + (static_cast<int64_t>(bq) * D + 2 * dp) * 4;
  };
  // Steps are fetched two ahead: step s+2's loads go out while step s is
  // computed, and step s+1, loaded during step s-1, is stored to LDS after it.
  // Two register sets alternate, so the loop is unrolled by two; every load and
  // store is issued unconditionally (past the last step they repeat the last
  // step's addresses into a buffer nobody reads), which keeps the compiler's
  // wait for step s+1 exact instead of a wait for every load in flight.
  const int nsteps = (kend_wg + kStep - 1) / kStep;
  // The block-table entries of a step (its block, and at bs 16 the block of
  // tokens 16..31) are read one iteration before the step's loads go out, by
  // vector loads issued ahead of the previous step's K/V loads: so they are
  // in registers by the time they are used, and waiting for them never waits
  // for a K/V load (the loads complete in order). A scalar load would be
  // waited for together with the LDS operations in flight.
  const auto trsrc = tile_rsrc(trow, a.mb * 4);
  struct Ent {
    int a, b;
  };
  auto load_ent = [&](int step) -> Ent {
    const int t0 = min(step, nsteps - 1) * kStep;
    const int ia = t0 / BS;
    const int ib = (BS == 16 && t0 + 16 < kend_wg) ? ia + 1 : ia;
    return Ent{static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(trsrc, 4 * ia, 0, 0)),
               BS == 16 ? static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(trsrc, 4 * ib, 0, 0))
                        : 0};
  };
  auto fetch = [&](const Ent& e, u32x4 (&pre)[kPer]) {  // step -> registers
    const int ia = __builtin_amdgcn_readfirstlane(e.a);
    const int ib = BS == 16 ? __builtin_amdgcn_readfirstlane(e.b) : ia;
    const uint16_t* bA = pool + clamp_block(ia, a.nb) * a.blk_elems;
    const uint16_t* bB = pool + clamp_block(ib, a.nb) * a.blk_elems;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      bool from_b;
      const int64_t off = piece_src(u, u * kThreads + static_cast<int>(threadIdx.x), from_b);
      pre[u] = ld16((from_b ? bB : bA) + off);
    }
  };
  // Pieces u < kPer / 2 of a thread are K pieces and the rest V pieces (the
  // first kChunks / 2 piece numbers are K's); deciding by u keeps the choice
  // out of the per-lane code.
  static_assert(kChunks / 2 == (kPer / 2) * kThreads, "K pieces are the first half of every thread's");
  auto stash = [&](int buf, const u32x4 (&pre)[kPer]) {  // registers -> LDS buffer
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = u * kThreads + static_cast<int>(threadIdx.x);
      if (u < kPer / 2) {
        *reinterpret_cast<u32x4*>(&lk[buf * kK + pc * 8]) = pre[u];
      } else {
        // 4 tokens of dims 2dp and 2dp+1 of quad half `w` of quad pair cp,
        // 8 bytes each. Adjacent lanes hold the two halves of the same dims,
        // so each store instruction fills whole 16-byte rows pairwise (a
        // 2-way bank pattern; one lane per row pair would be 8-way).
        const int pv = pc - kChunks / 2;
        const int m = pv >> 1, w = pv & 1;
        const int cp = m / (D / 2), dp = m - cp * (D / 2);
        uint16_t* row = &lv[buf * kV + (cp * D + 2 * dp) * 8 + w * 4];
        *reinterpret_cast<u32x2*>(row) = u32x2{pre[u][0], pre[u][1]};
        *reinterpret_cast<u32x2*>(row + 8) = u32x2{pre[u][2], pre[u][3]};
      }
    }
  };
  // One step from LDS: the K operands feed the scores, then the V operands are
  // read into registers the K operands no longer need while the softmax runs.
  // EDGE: the step may reach past the end of the keys or past some row's
  // limit (see PrefillEngine::edge_masks).
  auto step = [&]<bool EDGE>(int buf, int t0) {
    u32x4 kop[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      kop[s2] = *reinterpret_cast<const u32x4*>(&lk[buf * kK + ((2 * s2 + h) * kStep + r) * 8]);
    f32x16 sc = eng.scores(kop);
    // every K operand read goes out before the first score MFMA: the MFMAs
    // form one dependent chain, and a read issued just before its MFMA would
    // add an LDS latency to each link
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);  // MFMAs
    __builtin_amdgcn_sched_barrier(0);  // (the V reads below stay out of that group)
    u32x4 vv[2 * DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int mh = 0; mh < 2; ++mh)
        vv[2 * db + mh] =
            *reinterpret_cast<const u32x4*>(&lv[buf * kV + ((2 * mh + h) * D + 32 * db + r) * 8]);
    if constexpr (EDGE) eng.edge_masks(sc, vv, t0, kend_wg, h);
    eng.softmax_pv(sc, vv, a.sl2e);
  };
  // Iteration s: read the table entries of step s+3 and fetch step s+2 into
  // `fetch_into` (free: its step s went to LDS in iteration s-1), compute
  // step s from LDS buffer s&1, store step s+1 from `held` into LDS buffer
  // (s+1)&1 (last read in iteration s-1, before its barrier), then one
  // barrier.
  Ent ent_next;  // entries of step s+2 in iteration s
  auto iteration = [&]<bool EDGE>(int s, u32x4 (&fetch_into)[kPer], const u32x4 (&held)[kPer]) {
    const int t0 = s * kStep;
    const int buf = s & 1;
    const Ent e = ent_next;
    ent_next = load_ent(s + 3);
    fetch(e, fetch_into);
    if (s < nsteps && i0 < L && t0 < kend) step.template operator()<EDGE>(buf, t0);  // uniform
    stash((s + 1) & 1, held);
    __syncthreads();
  };
  u32x4 preA[kPer], preB[kPer];
  {
    const Ent e0 = load_ent(0), e1 = load_ent(1);
    ent_next = load_ent(2);
    fetch(e0, preA);
    fetch(e1, preB);
  }
  stash(0, preA);
  __syncthreads();
  // Steps before `inner` lie wholly before the end of the keys and at or
  // before every row's limit of the workgroup (whose smallest is that of its
  // first position), so they need no masks: a loop of their own keeps its
  // body free of the mask branches. The rest (about two steps of a tile) test
  // for masks as they go. Both loops take steps in pairs, as the register
  // sets alternate.
  const int inner = max(0, min(nsteps, (prior + wg_i0 + 1) / kStep)) & ~1;
  int s = 0;
  for (; s < inner; s += 2) {
    iteration.template operator()<false>(s, preA, preB);
    iteration.template operator()<false>(s + 1, preB, preA);
  }
  for (; s < nsteps; s += 2) {
    iteration.template operator()<true>(s, preA, preB);
    iteration.template operator()<true>(s + 1, preB, preA);
  }
  const float lt = eng.l + __shfl_xor(eng.l, 32);  // both halves of the row
  if (i >= L) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) +
                   ((static_cast<int64_t>(q0) + i) * a.hq + g * G + hd) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int p = 0; p < 4; ++p)
      store4<uint16_t>(orow + 32 * db + 8 * p + 4 * h,
                       f32x4{eng.o[db][4 * p], eng.o[db][4 * p + 1], eng.o[db][4 * p + 2],
                             eng.o[db][4 * p + 3]} * inv);
}

// One workgroup per tile, in grid order: (x, chunk, kv head) = blockIdx.
template <int D, int BS>
__global__ __launch_bounds__(64 * prefill_waves(D)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(PrefillArgs a) {
  __shared__ PrefillSmem<D> sm;
  prefill_tile<D, BS, prefill_waves(D)>(a, sm, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Tiles in longest-first order. A tile's work is its number of 32-token key
// steps, known from the chunk geometry alone, so every workgroup ranks the
// (chunk, x) tiles by it in LDS (ties: lower index first; the kv heads of one
// (chunk, x) follow each other). Round k hands tile k*P + w (k even) or
// k*P + P-1-w (k odd) to workgroup w: a serpentine deal of the sorted list,
// which keeps the longest tiles from ending up on the same workgroups.
constexpr int kMaxPrefillTiles = 1024;  // (chunk, x) pairs ranked in LDS

template <int D>
struct PrefillLds {
  PrefillSmem<D> sm;
  int key[kMaxPrefillTiles];    // key steps of (chunk, x) pair i = c * gx + x
  int order[kMaxPrefillTiles];  // pairs by decreasing key
  int next;
};

// Ranks the (chunk, x) pairs by their number of key steps; returns how many
// pairs there are. Ends with a barrier.
template <int BS, int W>
__device__ __forceinline__ int prefill_rank(const PrefillArgs& a, int gx, int* __restrict__ key_of,
                                            int* __restrict__ order) {
  const int M = a.num_chunks * gx;
  const int G = a.hq / a.hkv;
  const int pos_per_wg = W * kPrefillRows / G;
  for (int i = threadIdx.x; i < M; i += W * 64) {
    const int c = i / gx, x = i - c * gx;
    int q0, L, prior, key = 0;
    if (chunk_geometry(a, c, a.mb * BS, q0, L, prior) && x * pos_per_wg < L)
      key = (prior + min(L, (x + 1) * pos_per_wg) + kStep - 1) / kStep;
    key_of[i] = key;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < M; i += W * 64) {
    const int ki = key_of[i];
    int rank = 0;
    for (int j = 0; j < M; ++j) {
      const int kj = key_of[j];
      rank += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
    }
    order[rank] = i;
  }
  __syncthreads();
  return M;
}

template <int D, int BS>
__global__ __launch_bounds__(64 * prefill_waves(D)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_lpt_kernel(PrefillArgs a, int gx) {
  constexpr int W = prefill_waves(D);
  __shared__ PrefillSmem<D> sm;
  __shared__ int s_key[kMaxPrefillTiles];
  __shared__ int s_order[kMaxPrefillTiles];
  const int tiles = prefill_rank<BS, W>(a, gx, s_key, s_order) * a.hkv;
  const int P = static_cast<int>(gridDim.x);
  for (int k = 0; k * P < tiles; ++k) {
    const int t = k * P + ((k & 1) ? P - 1 - static_cast<int>(blockIdx.x)
                                   : static_cast<int>(blockIdx.x));
    if (t >= tiles) break;
    const int combo = s_order[t / a.hkv];
    if (s_key[combo] == 0) break;  // sorted: every later tile is empty too
    prefill_tile<D, BS, W>(a, sm, combo % gx, combo / gx, t % a.hkv);
  }
}

// ---------------------------------------------------------------------------
// Mixed batch: decode sequences and prefill chunks in one persistent launch.
//
// The workgroups share two work lists: decode items from the decode queue and
// prefill tiles, longest first, from a second counter. The grid holds two
// workgroups per CU; the first half of the grid (one per CU, as the
// dispatcher fills every CU's first slot before any second one) starts on
// prefill tiles and the second half on decode items, and each turns to the
// other list when its first one runs dry. So while both lists last, a CU
// holds one workgroup of each kind: the HBM-bound decode steps and the
// MFMA-bound prefill steps overlap instead of running back to back. The
// decode side merges the split-K partitions of long sequences itself.
// ---------------------------------------------------------------------------
template <int D>
union MixedSmem {
  DecodeSmem<D> d;
  PrefillLds<D> p;
};

template <int D, int BS>
__device__ __forceinline__ void prefill_from_queue(const PrefillArgs& a, int gx,
                                                   int32_t* __restrict__ queue,
                                                   PrefillLds<D>& ps) {
  const int tiles = prefill_rank<BS, kWaves>(a, gx, ps.key, ps.order) * a.hkv;
  for (;;) {
    if (threadIdx.x == 0) ps.next = atomicAdd(&queue[2], 1);
    __syncthreads();
    const int t = ps.next;
    __syncthreads();  // read before the next tile's thread 0 rewrites it
    if (t >= tiles) break;
    const int combo = ps.order[t / a.hkv];
    if (ps.key[combo] == 0) break;  // sorted: every later tile is empty too
    prefill_tile<D, BS, kWaves>(a, ps.sm, combo % gx, combo / gx, t % a.hkv);
  }
}

template <int D, int BS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mixed_bf16_kernel(DecodeArgs da, PrefillArgs pa, int gx, int32_t* __restrict__ queue) {
  __shared__ MixedSmem<D> u;
  const int half = gridDim.x / 2;
  const bool prefill_first = blockIdx.x < half;
  if (prefill_first) {
    if (pa.num_chunks > 0) prefill_from_queue<D, BS>(pa, gx, queue, u.p);
    __syncthreads();  // LDS changes hands
    if (da.num_seqs > 0) decode_persistent<D, BS>(da, queue, u.d, -1, gridDim.x - half);
  } else {
    // the decode-first half starts together: its first units are dealt
    if (da.num_seqs > 0)
      decode_persistent<D, BS>(da, queue, u.d, blockIdx.x - half, gridDim.x - half);
    __syncthreads();
    if (pa.num_chunks > 0) prefill_from_queue<D, BS>(pa, gx, queue, u.p);
  }
  leave_queue(queue);
}

// fp32: one workgroup per (position, chunk, kv head); its waves split the keys.
template <int D, int BS, int G>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs a) {
  const int i = blockIdx.x, c = blockIdx.y, g = blockIdx.z;
  int q0, L, prior;
  if (!chunk_geometry(a, c, a.mb * BS, q0, L, prior)) return;
  if (i >= L) return;
  __shared__ MergeSmem<D> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, cc = lane & 15;
  const float* pool = static_cast<const float*>(a.pool);
  const int64_t row0 = (static_cast<int64_t>(q0) + i) * a.hq + g * G;
  F32Engine<D, BS, G> eng;
  eng.init(static_cast<const float*>(a.q) + row0 * D, cc);
  const int kend = prior + i + 1;
  eng.lim = kend - 1;
  const int64_t kofs = static_cast<int64_t>(g) * BS * D;
  const int64_t vofs = static_cast<int64_t>(a.hkv) * BS * D + static_cast<int64_t>(g) * D * BS;
  const int32_t* trow = a.tables + static_cast<int64_t>(c) * a.mb;
  for (int t0 = wave * kStep; t0 < kend; t0 += kWaves * kStep) {
    int blkA, blkB;
    step_blocks<BS>(trow, t0, kend, a.nb, blkA, blkB);
    eng.step(pool, a.blk_elems, kofs, vofs, blkA, blkB, t0, kend, lane, a.sl2e);
  }
#pragma unroll
  for (int qi = 0; qi < G; ++qi) {
    const float lt = sum_over_groups(eng.l[qi]);
#pragma unroll
    for (int k = 0; k < F32Engine<D, BS, G>::EPL; ++k) {
      const float v = sum_over_groups(eng.acc[qi][k]);
      if (grp == 0) sm.o[wave][qi][cc + 16 * k] = v;
    }
    if (lane == 0) {
      sm.m[wave][qi] = eng.m[qi];
      sm.l[wave][qi] = lt;
    }
  }
  __syncthreads();
  finish_partition<D, float>(sm, G, 1, 0, static_cast<float*>(a.out) + row0 * D, nullptr,
                             nullptr);
}

// ---------------------------------------------------------------------------
// KV append and block copy (pure data movement).
// ---------------------------------------------------------------------------
// Wave -> (16 consecutive tokens of the list, kv head, 4 consecutive
// 8-element slices); lane -> (token lane/4, slice lane%4), so the four lanes
// of a token read 64 contiguous bytes of its row. Each lane loads its slot and
// its K and V slice in one round trip. K: the slice is one contiguous
// 8-element run at its slot, so lanes of consecutive slots write consecutive
// 16-byte pieces. V: the slice's 8 dimensions sit 4 elements apart in the
// token's 4-slot slice. When the four tokens holding slots 4j .. 4j+3 of one
// block are all in the wave (a prefill chunk's consecutive tokens are), the
// lane of the token at slot 4j+i gathers dimension pair i of all four tokens
// from the other three with lane shuffles and writes it as one contiguous
// piece, so the four write the slice's whole 8-dimension run; otherwise each
// lane writes its own token's V elements.
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kernel(T* __restrict__ pool,
                                                     const T* __restrict__ kn,
                                                     const T* __restrict__ vn,
                                                     const int32_t* __restrict__ slots,
                                                     int num_tokens, int hkv, int bs,
                                                     int64_t blk_elems, int64_t num_slots) {
  constexpr int CH = D / 8;
  constexpr int E16 = 16 / sizeof(T);    // elements per 16-byte word
  constexpr int W = 8 / E16;             // 16-byte words per 8-element slice
  constexpr int WPP = sizeof(T) / 2;     // 32-bit words per dimension pair
  constexpr int CG = CH / 4;             // groups of 4 slices
  static_assert(CH % 4 == 0, "a wave takes 4 slices of each token");
  const int lane = threadIdx.x & 63;
  const int tl = lane >> 2, cl = lane & 3;  // token and slice within the wave
  const int64_t wid = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
  const int64_t per_blk = static_cast<int64_t>(hkv) * CG;
  const int64_t tb = wid / per_blk;
  const int rem = static_cast<int>(wid - tb * per_blk);
  const int h = rem / CG, ch = (rem - h * CG) * 4 + cl;
  const int64_t tok = tb * 16 + tl;
  const bool in = tok < num_tokens;
  // one round trip: the slot and this token's K and V slice
  const int64_t src = ((in ? tok : 0) * hkv + h) * D + ch * 8;
  u32x4 kw[W], vw[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    kw[w] = ld16(kn + src + w * E16);
    vw[w] = ld16(vn + src + w * E16);
  }
  const int slot = in ? slots[tok] : -1;
  const bool valid = slot >= 0 && slot < num_slots;
  const int64_t blk = valid ? slot / bs : 0;
  const int off = valid ? slot - static_cast<int>(blk) * bs : 0;
  const int64_t tile = static_cast<int64_t>(h) * bs * D;
  if (valid) {
    T* kd = pool + blk * blk_elems + tile + (static_cast<int64_t>(ch) * bs + off) * 8;
#pragma unroll
    for (int w = 0; w < W; ++w) st16(kd + w * E16, kw[w]);
  }
  // V. The tokens of one 4-slot slice: base .. base+3 of the wave with
  // base = tl - off%4. Every lane runs the shuffles (clamped indices); the
  // slice is whole iff those four tokens hold its four slots in order, which
  // all four lanes then see.
  const int r = off & 3;
  const int base = tl - r;
  bool quad = valid && base >= 0 && base + 3 < 16;
  uint32_t words[4 * W];  // this lane's 8 dimensions as 32-bit words
#pragma unroll
  for (int w = 0; w < W; ++w)
#pragma unroll
    for (int x = 0; x < 4; ++x) words[4 * w + x] = vw[w][x];
  uint32_t g[4][WPP] = {};  // dimension pair r of tokens base .. base+3
  // Waves whose slots never run on (a decode step's one token per sequence)
  // skip the shuffles: the test is uniform over the wave.
  const int next_slot = __shfl(slot, min(lane + 4, 63));  // the next token, same slice
  if (__builtin_amdgcn_ballot_w64(valid && tl < 15 && next_slot == slot + 1) != 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int from = min(max(base + j, 0), 15) * 4 + cl;
      quad = quad && __shfl(slot, from) == slot - r + j;
#pragma unroll
      for (int x = 0; x < WPP; ++x) {
        // the word of dimension pair r sits at index r*WPP + x of the
        // sender; every lane asks for its own r, so all four candidates are
        // gathered and the lane picks its own
        uint32_t pick = 0;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t c =
              static_cast<uint32_t>(__shfl(static_cast<int>(words[rr * WPP + x]), from));
          pick = (rr == r) ? c : pick;
        }
        g[j][x] = pick;
      }
    }
  } else {
    quad = false;
  }
  T* vslice = pool + blk * blk_elems + static_cast<int64_t>(hkv) * bs * D + tile +
              (static_cast<int64_t>(off / 4) * D + ch * 8) * 4;
  if (quad) {
    // dims 2r and 2r+1 of the four tokens: [dim 2r: t0 t1 t2 t3][dim 2r+1: t0 .. t3]
    T* dst = vslice + 8 * r;  // vslice is slot position 0 of dimension ch*8
    if constexpr (sizeof(T) == 2) {
      u32x4 o;
      o[0] = (g[0][0] & 0xFFFFu) | (g[1][0] << 16);
      o[1] = (g[2][0] & 0xFFFFu) | (g[3][0] << 16);
      o[2] = (g[0][0] >> 16) | (g[1][0] & 0xFFFF0000u);
      o[3] = (g[2][0] >> 16) | (g[3][0] & 0xFFFF0000u);
      st16(dst, o);
    } else {
      st16(dst, u32x4{g[0][0], g[1][0], g[2][0], g[3][0]});
      st16(dst + 4, u32x4{g[0][1], g[1][1], g[2][1], g[3][1]});
    }
  } else if (valid) {
    const T* v = reinterpret_cast<const T*>(words);
#pragma unroll
    for (int e = 0; e < 8; ++e) vslice[4 * e + r] = v[e];
  }
}

// Whole blocks from one pool to another (the same one for copy-on-write; the
// device pool and a pinned host pool for swapping): pair p copies block
// pairs[2p] of `from` onto block pairs[2p+1] of `to`.
__global__ __launch_bounds__(256) void copy_blocks_kernel(const uint8_t* __restrict__ from,
                                                          uint8_t* __restrict__ to,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t blk_bytes, int64_t nb_from,
                                                          int64_t nb_to) {
  const int pi = blockIdx.y;
  const int src = pairs[2 * pi], dst = pairs[2 * pi + 1];
  if (static_cast<uint32_t>(src) >= static_cast<uint64_t>(nb_from) ||
      static_cast<uint32_t>(dst) >= static_cast<uint64_t>(nb_to))
    return;
  const u32x4* s = reinterpret_cast<const u32x4*>(from + src * blk_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(to + dst * blk_bytes);
  const int64_t n16 = blk_bytes / 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a0 = s[i], a1 = s[i + stride], a2 = s[i + 2 * stride], a3 = s[i + 3 * stride];
    d[i] = a0;
    d[i + stride] = a1;
    d[i + 2 * stride] = a2;
    d[i + 3 * stride] = a3;
  }
  for (; i < n16; i += stride) d[i] = s[i];
}

// ---------------------------------------------------------------------------
// Dispatch helpers.
// ---------------------------------------------------------------------------
// Workgroups of `threads` threads that fit on the device at once for `kernel`
// (0 if unknown).
template <typename K>
int resident_workgroups(K kernel, int threads = 256) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 0;
  return cus * per_cu;
}

// Compute units of the current device (0 if unknown).
inline int compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

template <int D, int BS>
hipError_t launch_decode_bf16(const DecodeArgs& a, int grid, int32_t* queue, hipStream_t st) {
  if (a.num_seqs <= kMaxScanSeqs) {
    // One workgroup per compute unit, although two fit. Each wave keeps two
    // 16 KiB steps in flight; with a second workgroup per unit (about 64 MiB
    // in flight on an HBM-bound batch) the extra loads only lengthen the
    // queueing latency of every load, and the tail, where each workgroup waits
    // out its last items, stretches with it. Cached batches (shared prefixes,
    // small calls) gain from one per unit too. Measured, two per unit -> one:
    // GQA long-tail batch 244.8 -> 239.5 us, MHA batch 185.6 -> 181.6 us,
    // shared-prefix batch 192.8 -> 184.9 us, engine loop (paged) 1.44 -> 1.49 M
    // tokens/s.
    // The persistent kernel merges split-K partitions itself.
    static const int cus = compute_units();
    const int w = min(grid, cus > 0 ? cus : 256);
    if (a.k_new != nullptr)
      hipLaunchKernelGGL((decode_bf16_append_kernel<D, BS>), dim3(w), dim3(256), 0, st, a,
                         queue);
    else if (a.share != nullptr)
      hipLaunchKernelGGL((decode_bf16_shared_kernel<D, BS>), dim3(w), dim3(256), 0, st, a,
                         queue);
    else
      hipLaunchKernelGGL((decode_bf16_persistent_kernel<D, BS>), dim3(w), dim3(256), 0, st, a,
                         queue);
  } else {
    hipLaunchKernelGGL((decode_bf16_kernel<D, BS>), dim3(grid), dim3(256), 0, st, a);
    if (a.np_max > 1)
      hipLaunchKernelGGL((decode_merge_kernel<D, BS, uint16_t>), dim3(a.num_seqs * a.hkv),
                         dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_decode_f32(const DecodeArgs& a, int G, int grid, hipStream_t st) {
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_f32_kernel<D, BS, 1>), dim3(grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_f32_kernel<D, BS, 2>), dim3(grid), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_f32_kernel<D, BS, 4>), dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((decode_f32_kernel<D, BS, 8>), dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  if (a.np_max > 1)
    hipLaunchKernelGGL((decode_merge_kernel<D, BS, float>), dim3(a.num_seqs * a.hkv), dim3(256), 0,
                       st, a);
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_prefill_bf16(const PrefillArgs& a, int max_chunk_len, hipStream_t st) {
  const int G = a.hq / a.hkv;
  constexpr int W = prefill_waves(D);
  const int pos_per_wg = W * kPrefillRows / G;
  const int gx = (max_chunk_len + pos_per_wg - 1) / pos_per_wg;
  const int64_t combos = static_cast<int64_t>(gx) * a.num_chunks;
  if (combos <= kMaxPrefillTiles) {
    static const int resident = resident_workgroups(prefill_bf16_lpt_kernel<D, BS>, 64 * W);
    const int64_t tiles = combos * a.hkv;
    const int64_t cap = resident > 0 ? resident : 512;
    const int w = static_cast<int>(tiles < cap ? tiles : cap);
    hipLaunchKernelGGL((prefill_bf16_lpt_kernel<D, BS>), dim3(w), dim3(64 * W), 0, st,
                       a, gx);
  } else {
    dim3 grid(gx, a.num_chunks, a.hkv);
    hipLaunchKernelGGL((prefill_bf16_kernel<D, BS>), grid, dim3(64 * W), 0, st, a);
  }
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_prefill_f32(const PrefillArgs& a, int max_chunk_len, hipStream_t st) {
  const int G = a.hq / a.hkv;
  dim3 grid(max_chunk_len, a.num_chunks, a.hkv);
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_f32_kernel<D, BS, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_f32_kernel<D, BS, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((prefill_f32_kernel<D, BS, 4>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((prefill_f32_kernel<D, BS, 8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers (shapes already validated by the caller).
// ---------------------------------------------------------------------------
hipError_t launch_append(void* pool, const void* k_new, const void* v_new, const int32_t* slots,
                         int num_tokens, const PoolShape& ps, int dtype, hipStream_t st) {
  if (num_tokens == 0) return hipSuccess;
  // a wave per (16 tokens, kv head, 4 slices of 8 elements)
  const int64_t threads =
      (static_cast<int64_t>(num_tokens) + 15) / 16 * 64 * ps.num_kv_heads * (ps.head_dim / 32);
  const int grid = static_cast<int>((threads + 255) / 256);
  const int64_t num_slots = ps.num_blocks * ps.block_size;
  const int64_t be = ps.block_elems();
#define PA_APPEND(T, D)                                                                       \
  hipLaunchKernelGGL((append_kernel<T, D>), dim3(grid), dim3(256), 0, st, static_cast<T*>(pool), \
                     static_cast<const T*>(k_new), static_cast<const T*>(v_new), slots,          \
                     num_tokens, ps.num_kv_heads, ps.block_size, be, num_slots)
  if (dtype == 0) {
    if (ps.head_dim == 64) PA_APPEND(float, 64); else PA_APPEND(float, 128);
  } else {
    if (ps.head_dim == 64) PA_APPEND(uint16_t, 64); else PA_APPEND(uint16_t, 128);
  }
#undef PA_APPEND
  return hipGetLastError();
}

hipError_t launch_copy(void* pool, const int32_t* pairs, int num_pairs, const PoolShape& ps,
                       int dtype, hipStream_t st) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t blk_bytes = ps.block_elems() * (dtype == 0 ? 4 : 2);
  const int64_t n16 = blk_bytes / 16;
  int gx = static_cast<int>((n16 + 1023) / 1024);  // about 4 x 16 B per thread
  gx = gx < 1 ? 1 : gx;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, num_pairs), dim3(256), 0, st,
                     static_cast<const uint8_t*>(pool), static_cast<uint8_t*>(pool), pairs,
                     blk_bytes, ps.num_blocks, ps.num_blocks);
  return hipGetLastError();
}

hipError_t launch_swap(void* pool, void* host_dev, const int32_t* pairs, int num_pairs,
                       bool out, int64_t num_host_blocks, const PoolShape& ps, int dtype,
                       hipStream_t st) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t blk_bytes = ps.block_elems() * (dtype == 0 ? 4 : 2);
  const int64_t n16 = blk_bytes / 16;
  int gx = static_cast<int>((n16 + 1023) / 1024);
  gx = gx < 1 ? 1 : gx;
  const uint8_t* from = static_cast<const uint8_t*>(out ? pool : host_dev);
  uint8_t* to = static_cast<uint8_t*>(out ? host_dev : pool);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, num_pairs), dim3(256), 0, st, from, to, pairs,
                     blk_bytes, out ? ps.num_blocks : num_host_blocks,
                     out ? num_host_blocks : ps.num_blocks);
  return hipGetLastError();
}

namespace {

DecodeArgs decode_args(void* out, const void* q, const void* pool, const int32_t* tables,
                       const int32_t* lens, int num_seqs, int max_blocks_per_seq,
                       int max_context_len, int num_q_heads, const PoolShape& ps, float scale,
                       void* workspace, int32_t*& queue, size_t o_elem_bytes = sizeof(float)) {
  const int64_t np_max = decode_max_parts(max_context_len);
  const DecodeWorkspace wl =
      DecodeWorkspace::layout(num_seqs, num_q_heads, ps.head_dim, np_max, o_elem_bytes);
  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.pool = pool;
  a.tables = tables;
  a.lens = lens;
  a.num_seqs = num_seqs;
  a.mb = max_blocks_per_seq;
  a.hq = num_q_heads;
  a.hkv = ps.num_kv_heads;
  a.max_ctx = max_context_len;
  a.np_max = static_cast<int>(np_max);
  a.nb = ps.num_blocks;
  a.blk_elems = ps.block_elems();
  a.sl2e = scale * kLog2e;
  a.ws_o = static_cast<char*>(workspace) + wl.o_off;
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ml_off);
  queue = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + wl.queue_off);
  a.n_items = static_cast<int>(static_cast<int64_t>(num_seqs) * ps.num_kv_heads * np_max);
  a.share = nullptr;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.slots = nullptr;
  return a;
}

PrefillArgs prefill_args(void* out, const void* q, const void* pool, const int32_t* tables,
                         const int32_t* lens, const int32_t* qsl, int num_chunks,
                         int total_q_tokens, int max_blocks_per_seq, int num_q_heads,
                         const PoolShape& ps, float scale) {
  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.pool = pool;
  a.tables = tables;
  a.lens = lens;
  a.qsl = qsl;
  a.num_chunks = num_chunks;
  a.total_q = total_q_tokens;
  a.mb = max_blocks_per_seq;
  a.hq = num_q_heads;
  a.hkv = ps.num_kv_heads;
  a.nb = ps.num_blocks;
  a.blk_elems = ps.block_elems();
  a.sl2e = scale * kLog2e;
  return a;
}

template <int D, int BS>
hipError_t launch_mixed_bf16(const DecodeArgs& da, const PrefillArgs& pa, int gx, int32_t* queue,
                             hipStream_t st) {
  static const int resident = resident_workgroups(mixed_bf16_kernel<D, BS>);
  // (the persistent decode inside merges its split-K partitions itself)
  hipLaunchKernelGGL((mixed_bf16_kernel<D, BS>), dim3(resident > 0 ? resident : 512),
                     dim3(256), 0, st, da, pa, gx, queue);
  return hipGetLastError();
}

}  // namespace

// The allocation-free decode's workspace: one array per device, of fixed size,
// in the code object's own device memory. Host code never uses the array's
// name as an address (on the host it only names the symbol): its device
// address is looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

hipError_t dispatch_decode(const DecodeArgs& a, int32_t* queue, int num_q_heads,
                           const PoolShape& ps, int dtype, hipStream_t st) {
  const int grid = a.n_items;
  const int G = num_q_heads / ps.num_kv_heads;
  const int D = ps.head_dim, BS = ps.block_size;
  if (dtype == 1) {
    if (D == 64 && BS == 16) return launch_decode_bf16<64, 16>(a, grid, queue, st);
    if (D == 64 && BS == 32) return launch_decode_bf16<64, 32>(a, grid, queue, st);
    if (D == 128 && BS == 16) return launch_decode_bf16<128, 16>(a, grid, queue, st);
    if (D == 128 && BS == 32) return launch_decode_bf16<128, 32>(a, grid, queue, st);
  } else {
    if (D == 64 && BS == 16) return launch_decode_f32<64, 16>(a, G, grid, st);
    if (D == 64 && BS == 32) return launch_decode_f32<64, 32>(a, G, grid, st);
    if (D == 128 && BS == 16) return launch_decode_f32<128, 16>(a, G, grid, st);
    if (D == 128 && BS == 32) return launch_decode_f32<128, 32>(a, G, grid, st);
  }
  return hipErrorInvalidValue;
}

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up (and its queue
// counters cleared, on `st`) at the first call on that device; nullptr if the
// lookup fails.
void* scratch_on_current_device(hipStream_t st) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    // The counters start at zero with the code object; they are cleared once
    // more here by a kernel (not a memset), so that a caller capturing this
    // first call into a graph records an ordinary kernel node.
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, st, static_cast<uint32_t*>(p),
                       64);
    if (hipGetLastError() != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

hipError_t launch_decode(void* out, const void* q, const void* pool, const int32_t* tables,
                         const int32_t* lens, int num_seqs, int max_blocks_per_seq,
                         int max_context_len, int num_q_heads, const PoolShape& ps, float scale,
                         int dtype, void* workspace, hipStream_t st, const int32_t* share) {
  if (num_seqs == 0) return hipSuccess;
  int32_t* queue = nullptr;
  DecodeArgs a = decode_args(out, q, pool, tables, lens, num_seqs, max_blocks_per_seq,
                             max_context_len, num_q_heads, ps, scale, workspace, queue);
  a.share = share;  // (only the bf16 persistent decode reads it)
  return dispatch_decode(a, queue, num_q_heads, ps, dtype, st);
}

hipError_t launch_decode_append(void* out, const void* q, void* pool, const int32_t* tables,
                                const int32_t* lens, const void* k_new, const void* v_new,
                                const int32_t* slots, int num_seqs, int max_blocks_per_seq,
                                int max_context_len, int num_q_heads, const PoolShape& ps,
                                float scale, int dtype, void* workspace, hipStream_t st) {
  if (num_seqs == 0) return hipSuccess;
  if (dtype == 1 && num_seqs <= kMaxScanSeqs) {  // one launch
    int32_t* queue = nullptr;
    DecodeArgs a = decode_args(out, q, pool, tables, lens, num_seqs, max_blocks_per_seq,
                               max_context_len, num_q_heads, ps, scale, workspace, queue);
    a.k_new = k_new;
    a.v_new = v_new;
    a.slots = slots;
    return dispatch_decode(a, queue, num_q_heads, ps, dtype, st);
  }
  // otherwise the append, then the decode, on the same stream
  if (hipError_t e = launch_append(pool, k_new, v_new, slots, num_seqs, ps, dtype, st)) return e;
  return launch_decode(out, q, pool, tables, lens, num_seqs, max_blocks_per_seq, max_context_len,
                       num_q_heads, ps, scale, dtype, workspace, st);
}

hipError_t launch_decode_noalloc(void* out, const void* q, const void* pool, const int32_t* tables,
                                 const int32_t* lens, int num_seqs, int max_blocks_per_seq,
                                 int max_context_len, int num_q_heads, const PoolShape& ps,
                                 float scale, int dtype, hipStream_t st) {
  if (num_seqs == 0) return hipSuccess;
  void* ws = scratch_on_current_device(st);
  if (ws == nullptr) return hipErrorInvalidSymbol;
  int32_t* queue = nullptr;
  const DecodeArgs a =
      decode_args(out, q, pool, tables, lens, num_seqs, max_blocks_per_seq, max_context_len,
                  num_q_heads, ps, scale, ws, queue, dtype == 0 ? sizeof(float) : sizeof(uint16_t));
  return dispatch_decode(a, queue, num_q_heads, ps, dtype, st);
}

hipError_t launch_prefill(void* out, const void* q, const void* pool, const int32_t* tables,
                          const int32_t* lens, const int32_t* qsl, int num_chunks,
                          int total_q_tokens, int max_chunk_len, int max_blocks_per_seq,
                          int num_q_heads,
                          const PoolShape& ps, float scale, int dtype, hipStream_t st) {
  if (num_chunks == 0 || max_chunk_len == 0) return hipSuccess;
  const PrefillArgs a = prefill_args(out, q, pool, tables, lens, qsl, num_chunks, total_q_tokens,
                                     max_blocks_per_seq, num_q_heads, ps, scale);
  const int D = ps.head_dim, BS = ps.block_size;
  if (dtype == 1) {
    if (D == 64 && BS == 16) return launch_prefill_bf16<64, 16>(a, max_chunk_len, st);
    if (D == 64 && BS == 32) return launch_prefill_bf16<64, 32>(a, max_chunk_len, st);
    if (D == 128 && BS == 16) return launch_prefill_bf16<128, 16>(a, max_chunk_len, st);
    if (D == 128 && BS == 32) return launch_prefill_bf16<128, 32>(a, max_chunk_len, st);
  } else {
    if (D == 64 && BS == 16) return launch_prefill_f32<64, 16>(a, max_chunk_len, st);
    if (D == 64 && BS == 32) return launch_prefill_f32<64, 32>(a, max_chunk_len, st);
    if (D == 128 && BS == 16) return launch_prefill_f32<128, 16>(a, max_chunk_len, st);
    if (D == 128 && BS == 32) return launch_prefill_f32<128, 32>(a, max_chunk_len, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mixed(void* dec_out, const void* dec_q, const void* pool,
                        const int32_t* dec_tables, const int32_t* dec_lens, int num_seqs,
                        int dec_max_blocks, int max_context_len, void* pre_out,
                        const void* pre_q, const int32_t* pre_tables, const int32_t* pre_lens,
                        const int32_t* qsl, int num_chunks, int total_q_tokens, int max_chunk_len,
                        int pre_max_blocks, int num_q_heads, const PoolShape& ps, float scale,
                        int dtype, void* workspace, hipStream_t st) {
  const int G = num_q_heads / ps.num_kv_heads;
  const int pos_per_wg = kWaves * kPrefillRows / G;
  const int64_t gx = num_chunks > 0 ? (max_chunk_len + pos_per_wg - 1) / pos_per_wg : 0;
  const bool fused = dtype == 1 && num_seqs <= kMaxScanSeqs && gx * num_chunks <= kMaxPrefillTiles;
  if (!fused || num_seqs == 0 || num_chunks == 0 || max_chunk_len == 0) {
    // one kind of work only, or shapes the fused kernel does not take: the
    // two launches in turn
    if (hipError_t e = launch_decode(dec_out, dec_q, pool, dec_tables, dec_lens, num_seqs,
                                     dec_max_blocks, max_context_len, num_q_heads, ps, scale,
                                     dtype, workspace, st))
      return e;
    return launch_prefill(pre_out, pre_q, pool, pre_tables, pre_lens, qsl, num_chunks,
                          total_q_tokens, max_chunk_len, pre_max_blocks, num_q_heads, ps, scale,
                          dtype, st);
  }
  int32_t* queue = nullptr;
  const DecodeArgs da =
      decode_args(dec_out, dec_q, pool, dec_tables, dec_lens, num_seqs, dec_max_blocks,
                  max_context_len, num_q_heads, ps, scale, workspace, queue);
  const PrefillArgs pa = prefill_args(pre_out, pre_q, pool, pre_tables, pre_lens, qsl, num_chunks,
                                      total_q_tokens, pre_max_blocks, num_q_heads, ps, scale);
  const int D = ps.head_dim, BS = ps.block_size, gxi = static_cast<int>(gx);
  if (D == 64 && BS == 16) return launch_mixed_bf16<64, 16>(da, pa, gxi, queue, st);
  if (D == 64 && BS == 32) return launch_mixed_bf16<64, 32>(da, pa, gxi, queue, st);
  if (D == 128 && BS == 16) return launch_mixed_bf16<128, 16>(da, pa, gxi, queue, st);
  if (D == 128 && BS == 32) return launch_mixed_bf16<128, 32>(da, pa, gxi, queue, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
