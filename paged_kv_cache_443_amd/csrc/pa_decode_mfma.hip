// Paged decode attention on the CDNA4 matrix cores (bf16, int8 and int4 KV caches).
//
// What is computed (page "字节跳动 AI Infra (2)", KV-cache question, step-t
// equations): for each sequence and query head, softmax(scale * q . k_t)
// over the cached tokens t < L, applied to the v_t; the tokens are found
// through the block table (same page, PagedAttention kernel sketch), and
// the query heads of one GQA group share a K/V head (page "LLM推理优化",
// section 1.3).  The softmax is accumulated online, chunk by chunk, with
// running max / sum statistics (page "LLM推理优化", section 2: tiles of K/V
// are brought on chip, softmax statistics are updated per tile and the
// output accumulated, so no full score vector is stored); the KV-split form
// (FlashDecoding, page "字节跳动 AI Infra (2)", third question) writes per-
// partition normalised outputs and log-sum-exps instead of the final row.
//
// Work decomposition.  One work-group (NW wavefronts) per (kv head, group of
// <= 16 query heads, sequence[, partition]).  The wavefronts interleave over
// chunks of CT consecutive tokens (32 for bf16, 64 for int8 and int4: 16 KiB
// and 8 KiB of K+V per chunk at head_dim 128), keep one chunk in flight while computing the
// previous one, and merge their softmax states through LDS at the end.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, wave64):
//   S^T[token][head] = K[token][:] . Q[head][:]   A = 16 K rows, B = Q^T
//   O^T[d][head]    += V^T[d][token] P^T[token][head]   A = V^T, B = P^T
// The query heads of the GQA group are the N dimension, so one K/V tile
// read from HBM serves all of them.  Lane (m = lane % 16, j = lane / 16):
//   - QK, row group q: A row m is token TPL*(m/4) + 4q + (m%4); the output
//     gives lane (j, head m) the scores of tokens TPL*j + 4q + i, i < 4;
//   - PV: the B operand of lane (j, head m) is P of tokens TPL*j + 8r + e,
//     exactly the scores that lane already holds, and the A operand of lane
//     (j, channel m) is V of those 8 tokens at one channel: one 16-byte load
//     in the token-grouped V layout.
// K's channel-grouped layout makes each QK A-operand 16 contiguous bytes too.
// P enters the matrix core as bf16 hi + lo parts (two products), so the
// probabilities keep ~16 significant bits; scores and accumulators are fp32.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa_append_row.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// KV cache storage kinds (template argument KV).
constexpr int kBf16 = 0;
constexpr int kInt8 = 1;
constexpr int kInt4 = 2;
template <int KV>
constexpr bool kQuant = KV != kBf16;  // codes + fp16 scales per (token, kv head)

// Growth of a row's running maximum (log2 units) that the online softmax
// absorbs without rescaling its accumulators (probabilities stay < 2^8).
constexpr float kLazyLog2 = 8.f;

// One K/V storage vector: 16 bytes (8 bf16 or 16 int8 values), or 8 bytes
// of 16 int4 codes.  int4 keeps the int8 lane mapping with half the bytes.
template <int KV>
struct KvVec {
  typedef u32x4 T;
};
template <>
struct KvVec<kInt4> {
  typedef u32x2 T;
};

// Sequences a persistent split launch can index from LDS (4 bytes each).
constexpr int kMaxPersistentSeqs = 4096;
static_assert(kMaxFusedSplitSeqs <= kMaxPersistentSeqs, "fused split batches take the persistent pass");
// Sequences a single-pass launch ranks by length in every work-group (the
// ranking costs num_seqs^2 / threads LDS reads per work-group).
constexpr int kMaxLptSeqs = 512;

template <int KV, int D>
struct Tile {
  static constexpr int X = kQuant<KV> ? 16 : 8;    // elements per storage vector
  static constexpr int TPL = kQuant<KV> ? 16 : 8;  // tokens per lane group per chunk
  static constexpr int CT = 4 * TPL;         // tokens per chunk
  static constexpr int NQ = CT / 16;         // QK row groups per chunk
  static constexpr int NS = D / 32;          // MFMA k-steps over head_dim
  static constexpr int NKL = D / (4 * X);    // K vector loads per lane per row group
  static constexpr int ND = D / 16;          // 16-channel blocks of the output
  static constexpr int NR = TPL / 8;         // PV products per channel block
};

// Registers one chunk occupies while its loads are in flight.
// K of the next chunk is loaded while this chunk's softmax still runs, so
// everything the softmax reads besides the scores (the int8 scales) travels
// with the V buffer, which stays live until the chunk is finished.
template <int KV, int D>
struct KBuf {
  typename KvVec<KV>::T k[Tile<KV, D>::NQ][Tile<KV, D>::NKL];
};
template <int KV, int D>
struct VBuf {
  u32x4 ks[kQuant<KV> ? 2 : 1];  // int8 / int4: this lane group's 16 K scales
  u32x4 vs[kQuant<KV> ? 2 : 1];  // int8 / int4: this lane group's 16 V scales
  typename KvVec<KV>::T v[Tile<KV, D>::ND];
};

// Physical block ids this lane needs for one chunk (its K rows and its V tokens).
struct Ids {
  int32_t k, v;
};

template <int KV, int D, int BS>
struct Ctx {
  const typename KvVec<KV>::T *kpool;
  const typename KvVec<KV>::T *vpool;
  const u32x4 *kscale;   // int8 / int4 only: fp16 scales viewed as 16-byte vectors
  const u32x4 *vscale;
  const int32_t *tbl;    // LDS copy of the block-table window
  int32_t lb0;           // logical block of tbl[0]
  int32_t nbv;           // logical blocks holding positions < t1
  int32_t num_blocks_m1;
  int32_t kvh;
  int32_t hkv;
  int32_t t1;       // end of the token range (positions >= t1 are never used)
  int32_t t1_row;   // causal multi-query: this lane's query row sees positions < t1_row
  int32_t t1_min;   // causal multi-query: the smallest t1_row of the unit
  int32_t m, j;
  // fused append: position whose K and V come from the new row rather than
  // the cache (-1: none), and that row as this lane holds it: channels
  // 2*lane, 2*lane + 1 (head_dim 128) or channel lane (64), as bf16 bits,
  // int8 codes (a byte each, the lower channel first) or int4 codes (a nibble
  // each, the lower channel in the low nibble); int8 / int4: the row's K
  // scale (low half of news) and V scale (high half), fp16 bits
  int32_t newpos;
  int32_t newblk;  // fused append: the physical block slot_mapping names for the new row
  uint32_t newk, newv, news;
  uint8_t *scr;  // fused append: this wavefront's LDS merge slot, free while it streams
};

// K/V tile loads.  Tiles are read once per step and streamed past the caches
// (non-temporal) wherever a load instruction covers whole 128-byte lines, so
// that nothing is fetched twice: every bf16 load (K slot order above) and
// every V load.  int8 (int4) K row groups cover quarter (eighth) lines; the
// four row-group loads of a chunk share those lines, so quantised K uses
// ordinary loads and the lines stay in L2 between them.
template <bool STREAM, typename V>
__device__ __forceinline__ V load_tile(const V *ptr) {
  if constexpr (STREAM)
    return __builtin_nontemporal_load(ptr);
  else
    return *ptr;
}

// Block ids of chunk starting at position cs, read from the LDS table window.
template <int KV, int D, int BS>
__device__ __forceinline__ Ids read_ids(const Ctx<KV, D, BS> &x, int cs) {
  using T = Tile<KV, D>;
  // chunk starts are >= 0: unsigned division is a shift
  const int lbk = min(static_cast<int>(static_cast<uint32_t>(cs + T::TPL * (x.m >> 2)) / BS), x.nbv - 1) - x.lb0;
  const int lbv = min(static_cast<int>(static_cast<uint32_t>(cs + T::TPL * x.j) / BS), x.nbv - 1) - x.lb0;
  Ids r;
  // out-of-range ids are clamped so that a bad table can never fault
  r.k = static_cast<int32_t>(min(static_cast<uint32_t>(x.tbl[lbk]), static_cast<uint32_t>(x.num_blocks_m1)));
  r.v = static_cast<int32_t>(min(static_cast<uint32_t>(x.tbl[lbv]), static_cast<uint32_t>(x.num_blocks_m1)));
  return r;
}

// NT: non-temporal loads where they pay (every unit reads its K/V once);
// ordinary loads when several row groups of a unit read the same lines, so
// that the later reads hit the cache.
template <bool NT, int KV, int D, int BS>
__device__ __forceinline__ void issue_k(KBuf<KV, D> &kb, const Ctx<KV, D, BS> &x, int cs, Ids id) {
  using T = Tile<KV, D>;
  const size_t ktile = static_cast<size_t>(static_cast<uint32_t>(id.k) * static_cast<uint32_t>(x.hkv) + x.kvh);
  // K: [tile][D/X][BS] storage vectors
  const typename KvVec<KV>::T *kp = x.kpool + ktile * (D / T::X) * BS;
#pragma unroll
  for (int q = 0; q < T::NQ; ++q) {
    // chunk starts are multiples of 16 (windows, partitions and chunks are
    // multiples of the block size and of 16 tokens), so the 16-token slot
    // order depends on the lane's own offset only
    const int lt = T::TPL * (x.m >> 2) + 4 * q + (x.m & 3);
    const uint32_t off = static_cast<uint32_t>(cs + lt) % BS;
    const int ok = kQuant<KV> ? static_cast<int>(off) : static_cast<int>(off & ~15u) | bf16_k_slot(lt & 15);
#pragma unroll
    for (int s = 0; s < T::NKL; ++s) kb.k[q][s] = load_tile<NT && !kQuant<KV>>(kp + (4 * s + x.j) * BS + ok);
  }
}

template <bool NT, int KV, int D, int BS>
__device__ __forceinline__ void issue_v(VBuf<KV, D> &vb, const Ctx<KV, D, BS> &x, int cs, Ids id) {
  using T = Tile<KV, D>;
  const size_t vtile = static_cast<size_t>(static_cast<uint32_t>(id.v) * static_cast<uint32_t>(x.hkv) + x.kvh);
  // V: [tile][BS/X][D] storage vectors
  const int ov = static_cast<int>(static_cast<uint32_t>(cs + T::TPL * x.j) % BS);
  if constexpr (kQuant<KV>) {
    // scales first: the softmax needs them before PV needs the V data
    const size_t sidx = (vtile * BS + ov) / 8;
    vb.ks[0] = x.kscale[sidx];
    vb.ks[1] = x.kscale[sidx + 1];
    vb.vs[0] = x.vscale[sidx];
    vb.vs[1] = x.vscale[sidx + 1];
  }
  const typename KvVec<KV>::T *vp = x.vpool + (vtile * (BS / T::X) + ov / T::X) * D + x.m;
#pragma unroll
  for (int n = 0; n < T::ND; ++n) vb.v[n] = load_tile<NT>(vp + 16 * n);
}

// 32-bit words in one storage vector, and bits per element.
template <int KV>
constexpr int kVecWords = KV == kInt4 ? 2 : 4;
template <int KV>
constexpr int kElemBits = KV == kBf16 ? 16 : (KV == kInt8 ? 8 : 4);

// The new row staged in the wavefront's LDS slot as a storage vector holds
// it: K then V, D elements each (bf16 bits, int8 codes, or int4 codes two
// per byte with the even channel in the low nibble).  Every lane writes its
// channels (int4 at head_dim 64: even lanes write their pair's byte).
template <int KV, int D, int BS>
__device__ __forceinline__ void stage_new_row(const Ctx<KV, D, BS> &x, int lane) {
  constexpr int RB = D * kElemBits<KV> / 8;  // bytes of one row
  if constexpr (KV == kInt4 && D == 64) {
    const uint32_t k2 = (x.newk & 0xfu) | ((__shfl_xor(x.newk, 1) & 0xfu) << 4);
    const uint32_t v2 = (x.newv & 0xfu) | ((__shfl_xor(x.newv, 1) & 0xfu) << 4);
    if ((lane & 1) == 0) {
      x.scr[lane >> 1] = static_cast<uint8_t>(k2);
      x.scr[RB + (lane >> 1)] = static_cast<uint8_t>(v2);
    }
  } else {
    constexpr int LB = RB / 64;  // bytes per lane: 1, 2 or 4
    if constexpr (LB == 4) {
      reinterpret_cast<uint32_t *>(x.scr)[lane] = x.newk;
      reinterpret_cast<uint32_t *>(x.scr + RB)[lane] = x.newv;
    } else if constexpr (LB == 2) {
      reinterpret_cast<uint16_t *>(x.scr)[lane] = static_cast<uint16_t>(x.newk);
      reinterpret_cast<uint16_t *>(x.scr + RB)[lane] = static_cast<uint16_t>(x.newv);
    } else {
      x.scr[lane] = static_cast<uint8_t>(x.newk);
      x.scr[RB + lane] = static_cast<uint8_t>(x.newv);
    }
  }
}

// Replace element e (ELEM-bit elements) of a vector of NW 32-bit words.
template <int ELEM, int NW, typename Vec>
__device__ __forceinline__ void set_elem(Vec &v, int e, uint32_t val, bool hit) {
  constexpr int PERW = 32 / ELEM;
  const int k = e / PERW;
  const int sh = ELEM * (e % PERW);
  const uint32_t mask = ((1u << ELEM) - 1u) << sh;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (hit && w == k) v[w] = (v[w] & ~mask) | ((val << sh) & mask);
}

// K fragments of chunk cs: the lanes whose token is x.newpos take the new
// row's channels from the staged row (the bits the cache row will hold).
template <int KV, int D, int BS>
__device__ __forceinline__ void patch_new_k(KBuf<KV, D> &kb, const Ctx<KV, D, BS> &x, int cs) {
  using T = Tile<KV, D>;
  using Vec = typename KvVec<KV>::T;
#pragma unroll
  for (int q = 0; q < T::NQ; ++q) {
    const int t = cs + T::TPL * (x.m >> 2) + 4 * q + (x.m & 3);
    if (t == x.newpos) {
#pragma unroll
      for (int s = 0; s < T::NKL; ++s)  // this lane's vector: channels X * (4s + j) ..
        kb.k[q][s] = *reinterpret_cast<const Vec *>(x.scr + T::X * (4 * s + x.j) * kElemBits<KV> / 8);
    }
  }
}

// The V vectors of a lane group starting at tok0 (element newpos - tok0 of
// channel m + 16n takes the staged row's value) and, int8 / int4, the K and
// V scales of that token.
template <int KV, int D, int BS>
__device__ __forceinline__ void patch_new_v(VBuf<KV, D> &vb, const Ctx<KV, D, BS> &x, int tok0) {
  using T = Tile<KV, D>;
  constexpr int RB = D * kElemBits<KV> / 8;
  const int e = x.newpos - tok0;
  if (e >= 0 && e < T::X) {
#pragma unroll
    for (int n = 0; n < T::ND; ++n) {
      const int c = x.m + 16 * n;
      uint32_t val;
      if constexpr (KV == kBf16)
        val = reinterpret_cast<const uint16_t *>(x.scr + RB)[c];
      else if constexpr (KV == kInt8)
        val = x.scr[RB + c];
      else
        val = (x.scr[RB + (c >> 1)] >> (4 * (c & 1))) & 0xfu;
      set_elem<kElemBits<KV>, kVecWords<KV>>(vb.v[n], e, val, true);
    }
    if constexpr (kQuant<KV>) {
      // scales of tokens tok0 + 8i .. tok0 + 8i + 7 sit in ks[i] / vs[i]
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool in = (e >> 3) == i;
        set_elem<16, 4>(vb.ks[i], e & 7, x.news & 0xffffu, in);
        set_elem<16, 4>(vb.vs[i], e & 7, x.news >> 16, in);
      }
    }
  }
}

template <int KV, int D>
struct Scores {
  f32x4 s[Tile<KV, D>::NQ];  // row group q: tokens TPL*j + 4q + i of head m
};
template <int KV, int D>
struct Probs {
  float p[Tile<KV, D>::NQ * 4];  // tokens TPL*j + e of head m
};
template <int KV, int D>
struct QOp {
  bf16x8 q[Tile<KV, D>::NS];  // B operand of the QK product
  float bias;                 // int4: 136 * sum of the head's query, removed from its scores
};

template <int KV, int D>
struct State {
  f32x4 acc[Tile<KV, D>::ND];  // O^T[16n + 4j + i][head m]
  float m_run;                 // reference of the log2-domain exponentials (head m)
  float l_run;                 // this lane's share of the running sum
  float vsum;                  // int4: this lane's share of sum(p) fed to PV (same reference as acc)
};

// int4 caches: the K fragments carry 136 + code in even-first element order;
// give each query k-step the same order and keep 136 * sum(q) of the lane's
// head, which the scores lose again (the wavefront's lanes j of one head each
// hold a quarter of its channels).
template <int KV, int D>
__device__ __forceinline__ void prepare_qop(QOp<KV, D> &qop) {
  qop.bias = 0.f;
  if constexpr (KV == kInt4) {
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < Tile<KV, D>::NS; ++s) {
      qop.q[s] = __builtin_shufflevector(qop.q[s], qop.q[s], 0, 2, 4, 6, 1, 3, 5, 7);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += static_cast<float>(qop.q[s][e]);
    }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    qop.bias = kInt4Bias * sum;
  }
}

// int4 caches: remove 136 * sum(p) from every output of the lane's head (the
// V fragments carried 136 + code).
template <int KV, int D>
__device__ __forceinline__ void finish_state(State<KV, D> &st) {
  if constexpr (KV == kInt4) {
    float vs = st.vsum + __shfl_xor(st.vsum, 16);
    vs = vs + __shfl_xor(vs, 32);
    const float c = kInt4Bias * vs;
#pragma unroll
    for (int n = 0; n < Tile<KV, D>::ND; ++n) st.acc[n] -= c;
  }
}

// Scores of one chunk: S^T = K Q^T (row group q holds tokens TPL*j + 4q + i).
template <int KV, int D>
__device__ __forceinline__ void qk(Scores<KV, D> &S, const KBuf<KV, D> &kb, const QOp<KV, D> &qop) {
  using T = Tile<KV, D>;
#pragma unroll
  for (int q = 0; q < T::NQ; ++q) {
    S.s[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < T::NS; ++s) {
      bf16x8 a;
      if constexpr (KV == kInt8) {
        const u32x4 w = kb.k[q][s >> 1];
        a = (s & 1) ? i8x8_to_bf16x8(w[2], w[3]) : i8x8_to_bf16x8(w[0], w[1]);
      } else if constexpr (KV == kInt4) {
        const u32x2 w = kb.k[q][s >> 1];
        a = i4x8_to_bf16x8_biased((s & 1) ? w[1] : w[0]);
      } else {
        a = __builtin_bit_cast(bf16x8, kb.k[q][s]);
      }
      S.s[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop.q[s], S.s[q], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ float half_lo(uint32_t w) { return half_bits_to_float(static_cast<uint16_t>(w & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return half_bits_to_float(static_cast<uint16_t>(w >> 16)); }

// Online-softmax update for one chunk; returns the probabilities (V scale
// folded in for int8) of this lane's tokens TPL*j + e.  TAIL: positions may
// reach t1.
template <int KV, int D, bool TAIL, bool CAUSAL = false>
__device__ __forceinline__ void softmax(State<KV, D> &st, Scores<KV, D> &S, const VBuf<KV, D> &vb, Probs<KV, D> &P,
                                        int tok0, int t1, float scale_log2, float sbias) {
  using T = Tile<KV, D>;
  float mloc = -INFINITY;
#pragma unroll
  for (int q = 0; q < T::NQ; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * q + i;
      float sv;
      if constexpr (kQuant<KV>) {
        const uint32_t kw = vb.ks[e >> 3][(e >> 1) & 3];
        const float raw = KV == kInt4 ? S.s[q][i] - sbias : S.s[q][i];
        sv = raw * (scale_log2 * ((e & 1) ? half_hi(kw) : half_lo(kw)));
      } else {
        sv = S.s[q][i] * scale_log2;
      }
      if constexpr (TAIL) sv = (tok0 + e < t1) ? sv : -INFINITY;
      S.s[q][i] = sv;
      mloc = fmaxf(mloc, sv);
    }
  }
  mloc = max_over_rows(mloc);
  const float m_new = fmaxf(st.m_run, mloc);
  // The exponentials are taken against a reference (st.m_run) that moves only
  // when a chunk's maximum passes it by more than kLazyLog2, so every
  // probability stays below 2^kLazyLog2; only then are the accumulators
  // rescaled, and a wavefront whose rows all keep their reference skips the
  // rescale.  The result, acc / l, does not depend on the reference.
  const bool move = m_new > st.m_run + kLazyLog2;  // always, from -inf, once a position is seen
  const float ref = move ? m_new : st.m_run;
  // a causal query row may have seen no position yet: its reference is -inf
  // and the exponentials below must give 0, not NaN
  const float m_ref = (CAUSAL && ref == -INFINITY) ? 0.f : ref;
  const float alpha = move ? fast_exp2(st.m_run - m_new) : 1.f;
  st.m_run = ref;
  float psum = 0.f;
#pragma unroll
  for (int q = 0; q < T::NQ; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * q + i;
      const float pe = fast_exp2(S.s[q][i] - m_ref);
      psum += pe;
      if constexpr (kQuant<KV>) {
        const uint32_t vw = vb.vs[e >> 3][(e >> 1) & 3];
        float f = pe * ((e & 1) ? half_hi(vw) : half_lo(vw));  // V scale folded into P
        if constexpr (TAIL) f = (tok0 + e < t1) ? f : 0.f;     // scale of an unused slot may be NaN
        P.p[e] = f;
      } else {
        P.p[e] = pe;
      }
    }
  }
  st.l_run = st.l_run * alpha + psum;
  if constexpr (KV == kInt4) st.vsum *= alpha;
  if (__any(move)) {
#pragma unroll
    for (int n = 0; n < T::ND; ++n) st.acc[n] *= alpha;
  }
}

// O^T += V^T P^T, P split into bf16 hi + lo parts (LO), or P rounded to
// bf16 once (one product; the wide multi-query units).
template <int KV, int D, bool TAIL, bool LO = true>
__device__ __forceinline__ void pv_update(State<KV, D> &st, VBuf<KV, D> &vb, const Probs<KV, D> &P, int tok0,
                                          int t1) {
  using T = Tile<KV, D>;
  if constexpr (TAIL && !kQuant<KV>) {
    // V of positions >= t1 may hold NaN: zero it (0 * NaN would poison the sum)
    uint32_t keep[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      keep[k] = ((tok0 + 2 * k < t1) ? 0x0000ffffu : 0u) | ((tok0 + 2 * k + 1 < t1) ? 0xffff0000u : 0u);
#pragma unroll
    for (int n = 0; n < T::ND; ++n)
#pragma unroll
      for (int k = 0; k < 4; ++k) vb.v[n][k] &= keep[k];
  }
#pragma unroll
  for (int r = 0; r < T::NR; ++r) {
    bf16x8 phi, plo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // int4 V fragments hold their tokens even-first: P follows
      const float f = P.p[8 * r + (KV == kInt4 ? kEvenFirst[e] : e)];
      const __bf16 h = static_cast<__bf16>(f);
      phi[e] = h;
      if constexpr (LO) {
        const __bf16 lo = static_cast<__bf16>(f - static_cast<float>(h));
        plo[e] = lo;
        if constexpr (KV == kInt4) st.vsum += static_cast<float>(h) + static_cast<float>(lo);
      } else if constexpr (KV == kInt4) {
        st.vsum += static_cast<float>(h);
      }
    }
#pragma unroll
    for (int n = 0; n < T::ND; ++n) {
      bf16x8 a;
      if constexpr (KV == kInt8) {
        const u32x4 w = vb.v[n];
        a = r ? i8x8_to_bf16x8(w[2], w[3]) : i8x8_to_bf16x8(w[0], w[1]);
      } else if constexpr (KV == kInt4) {
        const u32x2 w = vb.v[n];
        a = i4x8_to_bf16x8_biased(r ? w[1] : w[0]);
      } else {
        a = __builtin_bit_cast(bf16x8, vb.v[n]);
      }
      st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, st.acc[n], 0, 0, 0);
      if constexpr (LO) st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, st.acc[n], 0, 0, 0);
    }
  }
}

// LDS of one work-group (dynamic: sized per launch by lds_bytes()):
//   int32 tbl[tbl_window]            block-table window
//   float m[NW][rows], l[NW][rows]   per-wavefront softmax statistics
//   float acc[NW][rows][D + 4]       per-wavefront output rows
//   int32 first[num_seqs + 1]        persistent split only: first piece of each sequence
// rows = min(16, group): only the query heads the work-group owns.
template <int D, int NW>
__host__ __device__ constexpr size_t lds_bytes(int tbl_window, int rows, int prefix_entries) {
  return static_cast<size_t>(tbl_window) * 4 + static_cast<size_t>(NW) * rows * (2 + D + 4) * 4 +
         static_cast<size_t>(prefix_entries) * 4;
}

struct Smem {
  int32_t *tbl;
  float *m;
  float *l;
  float *acc;
  int32_t *first;
};

template <int D, int NW>
__device__ __forceinline__ Smem carve(unsigned char *smem, int TW, int rows) {
  Smem sm;
  sm.tbl = reinterpret_cast<int32_t *>(smem);
  sm.m = reinterpret_cast<float *>(smem + static_cast<size_t>(TW) * 4);
  sm.l = sm.m + NW * rows;
  sm.acc = sm.l + NW * rows;  // [NW][rows][D + 4]
  sm.first = reinterpret_cast<int32_t *>(sm.acc + static_cast<size_t>(NW) * rows * (D + 4));
  return sm;
}

// Consume one chunk held in (kb, vb): QK, online softmax, PV.  With REFILL,
// the next loads into the same buffers are issued as soon as each buffer is
// read (K after QK, V after PV), for chunk `cn` with block ids `idn`.
// (sched_barrier pins the load issue points: left alone, the scheduler sinks
// them next to their first use and nothing stays in flight.)
// NEWROW (a chunk's tail, fused append): when the chunk holds x.newpos, that
// position's K and V (and int8 / int4 scales) come from the new row.
template <int KV, int D, int BS, bool TAIL, bool REFILL, bool CAUSAL = false, bool NT = true, bool NEWROW = false>
__device__ __forceinline__ void consume(State<KV, D> &st, KBuf<KV, D> &kb, VBuf<KV, D> &vb,
                                        const Ctx<KV, D, BS> &x, const QOp<KV, D> &qop, int cs, int cn, Ids idn,
                                        float scale_log2) {
  using T = Tile<KV, D>;
  Scores<KV, D> S;
  Probs<KV, D> P;
  bool spliced = false;
  if constexpr (NEWROW) {
    static_assert(TAIL && !REFILL, "the new row is spliced into a chunk's tail");
    // uniform over the wavefront: the chunk holds the new position, and the
    // table puts that position in the block the new row is written to
    spliced = x.newpos >= cs && x.newpos < cs + T::CT && x.tbl[x.newpos / BS - x.lb0] == x.newblk;
    if (spliced) {
      stage_new_row<KV, D, BS>(x, threadIdx.x & 63);  // a wavefront's LDS accesses are performed in order
      patch_new_k<KV, D, BS>(kb, x, cs);
    }
  }
  qk<KV, D>(S, kb, qop);
  if constexpr (NEWROW) {
    if (spliced) patch_new_v<KV, D, BS>(vb, x, cs + T::TPL * x.j);
  }
  if constexpr (REFILL) {
    __builtin_amdgcn_sched_barrier(0);
    issue_k<NT>(kb, x, cn, idn);
    __builtin_amdgcn_sched_barrier(0);
  }
  softmax<KV, D, TAIL, CAUSAL>(st, S, vb, P, cs + T::TPL * x.j, CAUSAL ? x.t1_row : x.t1, scale_log2, qop.bias);
  pv_update<KV, D, TAIL, KV != kInt4>(st, vb, P, cs + T::TPL * x.j, x.t1);
  if constexpr (REFILL) {
    __builtin_amdgcn_sched_barrier(0);
    issue_v<NT>(vb, x, cn, idn);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// A wavefront's n >= 1 chunks c_i = c0 + i * NW * CT with one chunk in flight
// while the previous one is computed.
template <int KV, int D, int BS, int NW, bool CAUSAL = false, bool NT = true, bool NEWROW = false>
__device__ __forceinline__ void stream_chunks(State<KV, D> &st, const Ctx<KV, D, BS> &x, const QOp<KV, D> &qop,
                                                int c0, int n, float scale_log2) {
  constexpr int STEP = NW * Tile<KV, D>::CT;
  KBuf<KV, D> kb;
  VBuf<KV, D> vb;
  int cs = c0;
  const Ids ids = read_ids(x, cs);
  issue_k<NT>(kb, x, cs, ids);
  issue_v<NT>(vb, x, cs, ids);
  for (int k = 0; k + 1 < n; ++k) {
    const int cn = cs + STEP;
    // a causal unit's last new tokens are hidden from its earlier query rows
    if (CAUSAL && cs + Tile<KV, D>::CT > x.t1_min)
      consume<KV, D, BS, true, true, CAUSAL, NT>(st, kb, vb, x, qop, cs, cn, read_ids(x, cn), scale_log2);
    else
      consume<KV, D, BS, false, true, CAUSAL, NT>(st, kb, vb, x, qop, cs, cn, read_ids(x, cn), scale_log2);
    cs = cn;
  }
  consume<KV, D, BS, true, false, CAUSAL, NT, NEWROW>(st, kb, vb, x, qop, cs, 0, Ids{0, 0},
                                                      scale_log2);  // may reach past t1
}

// One unit of work: (sequence b, kv head x query-head group hx[, partition]).
// Every thread of the work-group calls it with the same arguments.  On entry
// the LDS table window and merge buffers may be reused (the previous unit's
// readers are past its last barrier); on exit its outputs are written.
//
// Query rows.  The (query token, head) pairs a (sequence, kv head) serves are
// its rows: row r is query token r / G of the sequence with head
// kv * G + r % G.  A single-token decode has G rows (the GQA group); a causal
// multi-query unit has n_b * G.  Rows go to the matrix cores 16 at a time (a
// row group).  A unit takes R consecutive row groups of one kv head (`hx`
// names the kv head and the unit's first group / R): wavefront w serves row
// group w % R and takes every (NW / R)-th chunk of that group's tokens, so
// the R groups walk the same K/V chunks at about the same time and all but
// the first read of each line come from the cache.
template <int KV, int D, int BS, int NW, bool CAUSAL = false, int R = 1, bool FUSED = false, bool SHARED = false>
__device__ __forceinline__ void run_unit(const DecodeParams &p, const Smem &sm, int b, int hx, int part) {
  using T = Tile<KV, D>;
  static_assert(NW % R == 0, "row groups must divide the wavefronts");
  constexpr int NWT = NW / R;  // wavefronts sharing one row group's tokens
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wr = R == 1 ? 0 : w % R;
  const int wt = R == 1 ? w : w / R;
  const int kvh = hx / p.head_groups;
  const int rg0 = (hx % p.head_groups) * R;  // the unit's first row group
  const int r0 = (rg0 + wr) * 16;            // this wavefront's first row
  int nq = 1, qbase = b;  // query tokens of the sequence, index of its first one
  if constexpr (CAUSAL) {
    qbase = p.q_start[b];
    nq = p.q_start[b + 1] - qbase;
  }
  const int nrows = nq * p.group;
  // no row in the unit, or q_start out of its stated bounds: uniform over the
  // work-group, before any barrier
  if (CAUSAL && (rg0 * 16 >= nrows || qbase < 0 || qbase + nq > p.num_queries || nq > p.max_q_len)) return;
  const int gcount = min(16, nrows - r0);  // rows of this wavefront's group (<= 0: none)
  const int rows = p.rows_per_group;
  const int TW = p.tbl_window;
  const bool split = p.partition_size > 0;

  // ---- prologue: the length, the first block-table window and the queries are
  // independent loads, issued together -----------------------------------------
  const int32_t *table = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq;
  const int Lraw = p.context_lens[b];
  const int t0 = split ? part * p.partition_size : 0;
  const int lb_first = t0 / BS;
  {
    const int n_first = min(TW, p.max_blocks_per_seq - lb_first);
    for (int i = threadIdx.x; i < n_first; i += NW * 64) sm.tbl[i] = table[lb_first + i];
  }
  // fused append + decode (one unit per (sequence, kv head) or, split, per
  // (sequence, kv head, partition)): the sequence's new row for this kv head
  // is loaded here, alongside the table window, and used after the barrier
  // below (see there)
  static_assert(!FUSED || (!CAUSAL && R == 1), "the fused append needs one unit per (sequence, kv head)");
  AppendRowData<KV + 1, D> arow;
  if constexpr (FUSED) arow = load_append_row<KV + 1, D>(p.append, b, kvh, lane);
  const int L = min(max(Lraw, 0), p.max_blocks_per_seq * BS);
  // a partition past the end of its sequence is left untouched (uniform over
  // the work-group, and no barrier has been reached)
  if (split && t0 >= L) return;

  Ctx<KV, D, BS> x;
  x.m = lane & 15;
  x.j = lane >> 4;
  x.kvh = kvh;
  x.hkv = p.num_kv_heads;
  x.num_blocks_m1 = p.num_blocks - 1;
  x.kpool = static_cast<const typename KvVec<KV>::T *>(p.k_cache);
  x.vpool = static_cast<const typename KvVec<KV>::T *>(p.v_cache);
  x.kscale = reinterpret_cast<const u32x4 *>(p.k_scale);
  x.vscale = reinterpret_cast<const u32x4 *>(p.v_scale);
  x.tbl = sm.tbl;
  // the wavefront's own merge slot (rows * (D + 4) floats >= 2 * D * 2 bytes):
  // nothing reads or writes it until this wavefront has finished streaming
  x.scr = reinterpret_cast<uint8_t *>(sm.acc + static_cast<size_t>(w) * rows * (D + 4));

  // end of the positions read: a causal group's last row sees nothing past
  // its own position (none at all when nq > L: t1 <= 0).  x.t1 is this
  // wavefront's end, t1u the unit's (its last row group's).
  x.t1 = split ? min(t0 + p.partition_size, L) : L;
  int t1u = x.t1;
  if constexpr (CAUSAL) {
    const int r_last = min(nrows, (rg0 + R) * 16) - 1;
    t1u = min(x.t1, L - nq + r_last / p.group + 1);
    x.t1 = gcount > 0 ? min(x.t1, L - nq + (r0 + gcount - 1) / p.group + 1) : t0;
  } else if constexpr (R > 1) {
    if (gcount <= 0) x.t1 = t0;  // a row slot past the last query head
  }
  x.nbv = (x.t1 + BS - 1) / BS;
  x.newpos = -1;
  x.newblk = -1;
  x.newk = 0u;
  x.newv = 0u;
  x.news = 0u;

  // ---- query operand (B of the QK product): row r0 + m -------------------------
  QOp<KV, D> qop;
  {
    const int r = r0 + x.m;
    const int qi = CAUSAL ? r / p.group : 0;  // single-token rows are heads of query token 0
    const bool qvalid = x.m < gcount;
    const int hq = kvh * p.group + (CAUSAL ? r % p.group : r);
    const uint16_t *qrow =
        static_cast<const uint16_t *>(p.q) + (static_cast<size_t>(qbase + qi) * p.num_heads + hq) * D;
    // causal rows: query token qi sits at position L - nq + qi and sees the
    // positions up to it (lanes past the group's last row: up to t1); chunks
    // wholly before the group's first row's position need no mask
    x.t1_row = min(L - nq + qi + 1, x.t1);
    x.t1_min = L - nq + r0 / p.group + 1;
#pragma unroll
    for (int s = 0; s < T::NS; ++s) {
      const int d0 = kQuant<KV> ? (64 * (s >> 1) + 16 * x.j + 8 * (s & 1)) : (32 * s + 8 * x.j);
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (qvalid) v = *reinterpret_cast<const u32x4 *>(qrow + d0);
      qop.q[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  prepare_qop(qop);

  State<KV, D> st;
#pragma unroll
  for (int n = 0; n < T::ND; ++n) st.acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.vsum = 0.f;
  __syncthreads();  // first table window staged

  // Fused append.  The new token is position L - 1, in a block no other
  // sequence reads, so the only reader of its bytes is the wavefront whose
  // chunk holds L - 1.  Every wavefront holds the new row (int8 / int4:
  // quantised as the append quantises it, codes packed as the cache packs
  // them); the one whose last chunk holds L - 1 takes that position's K and
  // V (and scales) from it, the bits the cache row will hold, and nothing
  // here writes the cache: append work-groups do (append_rows).  A
  // wavefront's end, and any later wait on its memory counter, waits for its
  // stores to complete, a memory round trip that a unit here would add to
  // its time.
  if constexpr (FUSED) {
    const bool valid =
        L > 0 && arow.slot >= 0 && static_cast<int64_t>(arow.slot) < static_cast<int64_t>(p.num_blocks) * BS;
    if constexpr (KV == kBf16) {
      x.newk = arow.k.e[0];
      x.newv = arow.v.e[0];
      if constexpr (D == 128) {
        x.newk |= static_cast<uint32_t>(arow.k.e[1]) << 16;
        x.newv |= static_cast<uint32_t>(arow.v.e[1]) << 16;
      }
    } else {
      const QuantRow<D / 64> qr = quantize_row<KV + 1, D>(arow);  // whole wavefront
      if constexpr (KV == kInt8) {
        x.newk = static_cast<uint8_t>(qr.k.e[0]);
        x.newv = static_cast<uint8_t>(qr.v.e[0]);
        if constexpr (D == 128) {
          x.newk |= static_cast<uint32_t>(static_cast<uint8_t>(qr.k.e[1])) << 8;
          x.newv |= static_cast<uint32_t>(static_cast<uint8_t>(qr.v.e[1])) << 8;
        }
      } else {  // int4: a nibble per channel, the even channel low
        x.newk = static_cast<uint32_t>(qr.k.e[0]) & 0xfu;
        x.newv = static_cast<uint32_t>(qr.v.e[0]) & 0xfu;
        if constexpr (D == 128) {
          x.newk |= (static_cast<uint32_t>(qr.k.e[1]) & 0xfu) << 4;
          x.newv |= (static_cast<uint32_t>(qr.v.e[1]) & 0xfu) << 4;
        }
      }
      x.news = static_cast<uint32_t>(qr.sk) | (static_cast<uint32_t>(qr.sv) << 16);
    }
    // The row is spliced in only where the cache receives it: slot_mapping[b]
    // must be position L - 1's slot (its offset is checked here, its block
    // against the staged table entry where the splice happens).  Otherwise
    // position L - 1 is read from the cache, as pa_decode reads it after the
    // append, and the append work-groups write the row where the slot says.
    if (valid && arow.slot % BS == (L - 1) % BS) {
      x.newpos = L - 1;
      x.newblk = arow.slot / BS;
    }
  }

  // ---- token range in windows of staged block-table entries (usually one) ----
  for (int ws = t0; ws < t1u; ws += TW * BS) {
    const int we = min(ws + TW * BS, t1u);
    x.lb0 = ws / BS;
    if (ws != t0) {
      const int nbw = (we + BS - 1) / BS - x.lb0;
      __syncthreads();  // readers of the previous window are done
      for (int i = threadIdx.x; i < nbw; i += NW * 64) sm.tbl[i] = table[x.lb0 + i];
      __syncthreads();
    }

    // chunks ws + c*CT of this window below this wavefront's end; token share
    // wt takes c = wt, wt + NWT, ...
    const int wew = R == 1 ? we : min(we, x.t1);
    const int nch = wew > ws ? (wew - ws + T::CT - 1) / T::CT : 0;
    const int n = wt < nch ? (nch - wt + NWT - 1) / NWT : 0;
    if (n > 0)
      stream_chunks<KV, D, BS, NWT, CAUSAL, R == 1 && !SHARED, FUSED>(st, x, qop, ws + wt * T::CT, n,
                                                                      p.scale_log2);
  }

  // ---- merge the wavefronts' states -------------------------------------------
  finish_state(st);
  float l = st.l_run + __shfl_xor(st.l_run, 16);
  l = l + __shfl_xor(l, 32);
  if (x.m < rows) {
    float *arow = sm.acc + (static_cast<size_t>(w) * rows + x.m) * (D + 4);
#pragma unroll
    for (int n = 0; n < T::ND; ++n) *reinterpret_cast<f32x4 *>(arow + 16 * n + 4 * x.j) = st.acc[n];
    if (x.j == 0) {
      sm.m[w * rows + x.m] = st.m_run;
      sm.l[w * rows + x.m] = l;
    }
  }
  __syncthreads();

  // row group `slot` of the unit: states of wavefronts slot, slot + R, ...
#pragma unroll
  for (int slot = 0; slot < R; ++slot) {
    const int rs0 = (rg0 + slot) * 16;
    const int gc = R == 1 ? gcount : min(16, nrows - rs0);
    for (int e = threadIdx.x; e < gc * D; e += NW * 64) {
      const int gi = e / D;
      const int d = e % D;
      float M = -INFINITY;
#pragma unroll
      for (int t = 0; t < NWT; ++t) M = fmaxf(M, sm.m[(slot + t * R) * rows + gi]);
      float o = 0.f;
      float lse = -INFINITY;
      if (M != -INFINITY) {
        float lsum = 0.f, osum = 0.f;
#pragma unroll
        for (int t = 0; t < NWT; ++t) {
          const int v = slot + t * R;
          const float f = fast_exp2(sm.m[v * rows + gi] - M);
          lsum += f * sm.l[v * rows + gi];
          osum += f * sm.acc[(static_cast<size_t>(v) * rows + gi) * (D + 4) + d];
        }
        o = osum / lsum;
        lse = (M + __log2f(lsum)) * kLn2;
      }
      const int r = rs0 + gi;
      const int qi = CAUSAL ? r / p.group : 0;
      const int hq = kvh * p.group + (CAUSAL ? r % p.group : r);
      const size_t row = static_cast<size_t>(qbase + qi) * p.num_heads + hq;
      if (split) {
        const size_t prow = row * p.max_num_partitions + part;
        p.part_out[prow * D + d] = o;
        if (d == 0) p.part_lse[prow] = lse;
      } else if (p.out_bf16) {
        static_cast<uint16_t *>(p.out)[row * D + d] = float_to_bf16_bits(o);
      } else {
        static_cast<float *>(p.out)[row * D + d] = o;
      }
    }
  }
}

// Fused append + decode: the cache writes of the new rows.  The decode units splice each new row in from the source (run_unit),
// so no unit reads a row these writes touch and nothing orders them against
// the units.  Single pass: the grid's last work-groups write them, in the
// launch's tail where CUs free up; split pass: every persistent work-group
// writes its share after its last piece.  A wavefront writes
// kAppendRowsPerWave (token, kv head) rows at a time: all the loads first,
// then the stores.  One row per wavefront (more, shorter append work-groups)
// measured 0.7-1 us faster on the 70B-shaped step than four, neutral
// elsewhere.
constexpr int kAppendRowsPerWave = 1;

template <int KV, int D, int BS, int NW>
__device__ __forceinline__ void append_rows(const DecodeParams &p, int first_wg, int nwg) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rows = p.num_seqs * p.num_kv_heads;
  const int stride = nwg * NW;
  for (int r0 = first_wg * NW + w; r0 < rows; r0 += kAppendRowsPerWave * stride) {
    AppendRowData<KV + 1, D> rr[kAppendRowsPerWave];
#pragma unroll
    for (int k = 0; k < kAppendRowsPerWave; ++k) {
      const int r = r0 + k * stride;
      if (r < rows) rr[k] = load_append_row<KV + 1, D>(p.append, r / p.num_kv_heads, r % p.num_kv_heads, lane);
    }
#pragma unroll
    for (int k = 0; k < kAppendRowsPerWave; ++k) {
      const int r = r0 + k * stride;
      if (r < rows) store_append_row<KV + 1, D, BS>(p.append, rr[k], r % p.num_kv_heads, lane);
    }
  }
}

// ---- wide multi-query units ---------------------------------------------------
// When a (sequence, kv head) has many query rows (long chunked-prefill
// chunks), the narrow units above give each wavefront 16 rows and make every
// wavefront of a work-group fetch each K/V line from the cache for them.  A
// wide unit gives each wavefront RW row groups instead: every K/V fragment
// it loads feeds RW matrix-core products, so the cache traffic per product
// drops RW-fold.  Each wavefront walks its rows' whole token range alone and
// finishes its rows from registers (no LDS merge); the NW wavefronts of a
// work-group hold NW * RW consecutive row groups and read the same chunks at
// about the same time, so HBM sees each line about once per work-group.

// bf16 wide units: the scale is folded into the exponent's FMA (max taken on
// the raw scores; scale_log2 >= 0) and the row sums come from the matrix
// core (a ones operand against the same bf16 P as the PV product), so each
// lane holds its rows' whole sums in lsum.  With the loop-invariant address
// arithmetic, 512-token chunks on 64/8 heads 350.0 -> 333.0 us.
template <int D, bool TAIL>
__device__ __forceinline__ void softmax_fold(State<kBf16, D> &st, f32x4 &lsum, Scores<kBf16, D> &S,
                                             Probs<kBf16, D> &P, int tok0, int t1, float c) {
  using T = Tile<kBf16, D>;
  float mloc = -INFINITY;
#pragma unroll
  for (int q = 0; q < T::NQ; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * q + i;
      float sv = S.s[q][i];
      if constexpr (TAIL) sv = (tok0 + e < t1) ? sv : -INFINITY;
      S.s[q][i] = sv;
      mloc = fmaxf(mloc, sv);
    }
  }
  mloc = max_over_rows(mloc);
  const float mc = mloc == -INFINITY ? -INFINITY : mloc * c;
  const float m_new = fmaxf(st.m_run, mc);
  const bool move = m_new > st.m_run + kLazyLog2;
  const float ref = move ? m_new : st.m_run;
  const float nref = ref == -INFINITY ? 0.f : -ref;
  const float alpha = move ? fast_exp2(st.m_run - m_new) : 1.f;
  st.m_run = ref;
#pragma unroll
  for (int q = 0; q < T::NQ; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * q + i;
      float pe = fast_exp2(__builtin_fmaf(S.s[q][i], c, nref));
      if constexpr (TAIL) pe = (tok0 + e < t1) ? pe : 0.f;
      P.p[e] = pe;
    }
  }
  if (__any(move)) {
#pragma unroll
    for (int n = 0; n < T::ND; ++n) st.acc[n] *= alpha;
    lsum *= alpha;
  }
}

template <int D, bool TAIL>
__device__ __forceinline__ void pv_fold(State<kBf16, D> &st, f32x4 &lsum, VBuf<kBf16, D> &vb,
                                        const Probs<kBf16, D> &P, int tok0, int t1) {
  using T = Tile<kBf16, D>;
  static_assert(T::NR == 1, "one PV k-step per chunk");
  if constexpr (TAIL) {
    uint32_t keep[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      keep[k] = ((tok0 + 2 * k < t1) ? 0x0000ffffu : 0u) | ((tok0 + 2 * k + 1 < t1) ? 0xffff0000u : 0u);
#pragma unroll
    for (int n = 0; n < T::ND; ++n)
#pragma unroll
      for (int k = 0; k < 4; ++k) vb.v[n][k] &= keep[k];
  }
  bf16x8 ph;
#pragma unroll
  for (int e = 0; e < 8; ++e) ph[e] = static_cast<__bf16>(P.p[e]);
#pragma unroll
  for (int n = 0; n < T::ND; ++n)
    st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vb.v[n]), ph, st.acc[n], 0, 0, 0);
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ph, lsum, 0, 0, 0);
}

// One chunk of an int8 / int4 wide unit: QK, then each row group's softmax and PV.
template <int KV, int D, int BS, bool TAIL, bool REFILL, int RW>
__device__ __forceinline__ void consume_wide(State<KV, D> (&st)[RW], f32x4 (&lsum)[RW], KBuf<KV, D> &kb,
                                             VBuf<KV, D> &vb, const Ctx<KV, D, BS> &x, const QOp<KV, D> (&qop)[RW],
                                             const int (&t1r)[RW], int cs, int cn, Ids idn, float scale_log2) {
  static_assert(KV != kBf16, "bf16 wide units take consume_pipelined");
  using T = Tile<KV, D>;
  Scores<KV, D> S[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) qk<KV, D>(S[r], kb, qop[r]);
  if constexpr (REFILL) {
    __builtin_amdgcn_sched_barrier(0);
    issue_k<false>(kb, x, cn, idn);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    Probs<KV, D> P;
    softmax<KV, D, TAIL, true>(st[r], S[r], vb, P, cs + T::TPL * x.j, t1r[r], scale_log2, qop[r].bias);
    pv_update<KV, D, TAIL, false>(st[r], vb, P, cs + T::TPL * x.j, x.t1);
  }
  if constexpr (REFILL) {
    __builtin_amdgcn_sched_barrier(0);
    issue_v<false>(vb, x, cn, idn);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// bf16 wide units, software-pipelined over chunks: on entry S holds chunk
// cs's scores and kb holds K of the next chunk cn.  Chunk cn's QK products
// are issued before chunk cs's softmax and PV (they share no registers), so
// a wavefront's softmax never waits on the matrix-core results of its own
// chunk; K of chunk cnn (two ahead) then refills kb, V of cn refills vb once
// chunk cs's PV has read it.  Every product and its order is the same as
// in a chunk-by-chunk loop (QK, softmax, PV of one chunk, then the next), so
// the results are too, bit for bit.  NEXT: a chunk cn follows; REFILL: a
// chunk cnn follows it.
template <int D, int BS, bool TAIL, bool NEXT, bool REFILL, int RW>
__device__ __forceinline__ void consume_pipelined(State<kBf16, D> (&st)[RW], f32x4 (&lsum)[RW],
                                                  Scores<kBf16, D> (&S)[RW], KBuf<kBf16, D> &kb, VBuf<kBf16, D> &vb,
                                                  const Ctx<kBf16, D, BS> &x, const QOp<kBf16, D> (&qop)[RW],
                                                  const int (&t1r)[RW], int cs, int cn, Ids idn, int cnn, Ids idnn,
                                                  float scale_log2) {
  using T = Tile<kBf16, D>;
  Scores<kBf16, D> Sn[RW];
  if constexpr (NEXT) {
#pragma unroll
    for (int r = 0; r < RW; ++r) qk<kBf16, D>(Sn[r], kb, qop[r]);
    if constexpr (REFILL) {
      __builtin_amdgcn_sched_barrier(0);
      issue_k<false>(kb, x, cnn, idnn);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    Probs<kBf16, D> P;
    softmax_fold<D, TAIL>(st[r], lsum[r], S[r], P, cs + T::TPL * x.j, t1r[r], scale_log2);
    pv_fold<D, TAIL>(st[r], lsum[r], vb, P, cs + T::TPL * x.j, x.t1);
  }
  if constexpr (NEXT) {
    __builtin_amdgcn_sched_barrier(0);
    issue_v<false>(vb, x, cn, idn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RW; ++r) S[r] = Sn[r];
  }
}

// n >= 1 consecutive chunks from c0, the next one's loads in flight while
// the current one is computed (bf16: pipelined as above).
template <int KV, int D, int BS, int RW>
__device__ __forceinline__ void stream_wide(State<KV, D> (&st)[RW], f32x4 (&lsum)[RW], const Ctx<KV, D, BS> &x,
                                            const QOp<KV, D> (&qop)[RW], const int (&t1r)[RW], int c0, int n,
                                            float scale_log2) {
  constexpr int CT = Tile<KV, D>::CT;
  KBuf<KV, D> kb;
  VBuf<KV, D> vb;
  int cs = c0;
  const Ids ids = read_ids(x, cs);
  issue_k<false>(kb, x, cs, ids);
  issue_v<false>(vb, x, cs, ids);
  if constexpr (KV == kBf16) {
    Scores<KV, D> S[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) qk<KV, D>(S[r], kb, qop[r]);
    Ids idn{0, 0};  // block ids of chunk cs + CT, whose K is in flight
    if (n > 1) {
      idn = read_ids(x, cs + CT);
      issue_k<false>(kb, x, cs + CT, idn);
    }
    for (int k = 0; k + 1 < n; ++k) {
      const int cn = cs + CT;
      const int cnn = cn + CT;
      const bool tail = cs + CT > x.t1_min;  // the wavefront's first row cannot see all of chunk cs
      if (k + 2 < n) {
        const Ids idnn = read_ids(x, cnn);
        if (tail)
          consume_pipelined<D, BS, true, true, true, RW>(st, lsum, S, kb, vb, x, qop, t1r, cs, cn, idn, cnn, idnn,
                                                         scale_log2);
        else
          consume_pipelined<D, BS, false, true, true, RW>(st, lsum, S, kb, vb, x, qop, t1r, cs, cn, idn, cnn, idnn,
                                                          scale_log2);
        idn = idnn;
      } else {
        if (tail)
          consume_pipelined<D, BS, true, true, false, RW>(st, lsum, S, kb, vb, x, qop, t1r, cs, cn, idn, 0,
                                                          Ids{0, 0}, scale_log2);
        else
          consume_pipelined<D, BS, false, true, false, RW>(st, lsum, S, kb, vb, x, qop, t1r, cs, cn, idn, 0,
                                                           Ids{0, 0}, scale_log2);
      }
      cs = cn;
    }
    consume_pipelined<D, BS, true, false, false, RW>(st, lsum, S, kb, vb, x, qop, t1r, cs, 0, Ids{0, 0}, 0, Ids{0, 0},
                                                     scale_log2);
  } else {
    for (int k = 0; k + 1 < n; ++k) {
      const int cn = cs + CT;
      if (cs + CT > x.t1_min)  // the wavefront's first row cannot see all of this chunk
        consume_wide<KV, D, BS, true, true, RW>(st, lsum, kb, vb, x, qop, t1r, cs, cn, read_ids(x, cn), scale_log2);
      else
        consume_wide<KV, D, BS, false, true, RW>(st, lsum, kb, vb, x, qop, t1r, cs, cn, read_ids(x, cn), scale_log2);
      cs = cn;
    }
    consume_wide<KV, D, BS, true, false, RW>(st, lsum, kb, vb, x, qop, t1r, cs, 0, Ids{0, 0}, scale_log2);
  }
}

// One wide unit: sequence b, kv head hx / head_groups, row groups
// (hx % head_groups) * NW * RW + w * RW + r for wavefront w, r < RW.
template <int KV, int D, int BS, int NW, int RW>
__device__ __forceinline__ void run_wide_unit(const DecodeParams &p, int32_t *tbl, int b, int hx) {
  using T = Tile<KV, D>;
  constexpr int UNIT_ROWS = NW * RW * 16;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int kvh = hx / p.head_groups;
  const int ur0 = (hx % p.head_groups) * UNIT_ROWS;  // the unit's first row
  const int qbase = p.q_start[b];
  const int nq = p.q_start[b + 1] - qbase;
  const int nrows = nq * p.group;
  // uniform over the work-group, before any barrier
  if (ur0 >= nrows || qbase < 0 || qbase + nq > p.num_queries || nq > p.max_q_len) return;
  const int TW = p.tbl_window;
  const int32_t *table = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq;
  const int Lraw = p.context_lens[b];
  {
    const int n_first = min(TW, p.max_blocks_per_seq);
    for (int i = threadIdx.x; i < n_first; i += NW * 64) tbl[i] = table[i];
  }
  const int L = min(max(Lraw, 0), p.max_blocks_per_seq * BS);

  Ctx<KV, D, BS> x;
  x.m = lane & 15;
  x.j = lane >> 4;
  x.kvh = kvh;
  x.hkv = p.num_kv_heads;
  x.num_blocks_m1 = p.num_blocks - 1;
  x.kpool = static_cast<const typename KvVec<KV>::T *>(p.k_cache);
  x.vpool = static_cast<const typename KvVec<KV>::T *>(p.v_cache);
  x.kscale = reinterpret_cast<const u32x4 *>(p.k_scale);
  x.vscale = reinterpret_cast<const u32x4 *>(p.v_scale);
  x.tbl = tbl;
  x.newpos = -1;  // no fused append on wide units
  x.newblk = -1;
  x.newk = 0u;
  x.newv = 0u;
  x.news = 0u;
  x.scr = nullptr;

  // this wavefront's rows end at its last group's last row (none: t1 = 0);
  // the unit's at its last wavefront's
  const int wr0 = ur0 + w * RW * 16;
  const int t1u = min(L, L - nq + (min(nrows, ur0 + UNIT_ROWS) - 1) / p.group + 1);
  x.t1 = wr0 < nrows ? min(L, L - nq + (min(nrows, wr0 + RW * 16) - 1) / p.group + 1) : 0;
  x.nbv = (x.t1 + BS - 1) / BS;
  x.t1_min = L - nq + wr0 / p.group + 1;

  QOp<KV, D> qop[RW];
  int t1r[RW];
  int gc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int r0 = wr0 + 16 * r;
    gc[r] = min(16, nrows - r0);
    const int row = r0 + x.m;
    const int qi = row / p.group;
    const int hq = kvh * p.group + row % p.group;
    const bool qvalid = x.m < gc[r];
    const uint16_t *qrow =
        static_cast<const uint16_t *>(p.q) + (static_cast<size_t>(qbase + qi) * p.num_heads + hq) * D;
    t1r[r] = min(L - nq + qi + 1, x.t1);
#pragma unroll
    for (int s = 0; s < T::NS; ++s) {
      const int d0 = kQuant<KV> ? (64 * (s >> 1) + 16 * x.j + 8 * (s & 1)) : (32 * s + 8 * x.j);
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (qvalid) v = *reinterpret_cast<const u32x4 *>(qrow + d0);
      qop[r].q[s] = __builtin_bit_cast(bf16x8, v);
    }
    prepare_qop(qop[r]);
  }

  State<KV, D> st[RW];
  f32x4 lsum[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
#pragma unroll
    for (int n = 0; n < T::ND; ++n) st[r].acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    st[r].m_run = -INFINITY;
    st[r].l_run = 0.f;
    st[r].vsum = 0.f;
    lsum[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float scale_log2 = p.scale_log2;
  if constexpr (KV == kBf16) {
    // the folded exponent needs a scale >= 0: (-q) . k * (-scale) is the same score
    if (scale_log2 < 0.f) {
      scale_log2 = -scale_log2;
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int s2 = 0; s2 < T::NS; ++s2)
          qop[r].q[s2] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qop[r].q[s2]) ^ 0x80008000u);
    }
  }
  __syncthreads();  // first table window staged

  for (int ws = 0; ws < t1u; ws += TW * BS) {
    const int we = min(ws + TW * BS, t1u);
    x.lb0 = ws / BS;
    if (ws != 0) {
      const int nbw = (we + BS - 1) / BS - x.lb0;
      __syncthreads();  // readers of the previous window are done
      for (int i = threadIdx.x; i < nbw; i += NW * 64) tbl[i] = table[x.lb0 + i];
      __syncthreads();
    }
    const int wew = min(we, x.t1);
    if (wew > ws) stream_wide<KV, D, BS, RW>(st, lsum, x, qop, t1r, ws, (wew - ws + T::CT - 1) / T::CT, scale_log2);
  }

  // ---- finish this wavefront's rows from registers ----------------------------
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    finish_state(st[r]);
    float l = st[r].l_run + __shfl_xor(st[r].l_run, 16);
    l = l + __shfl_xor(l, 32);
    if constexpr (KV == kBf16) l = lsum[r][0];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (x.m < gc[r]) {
      const int row = wr0 + 16 * r + x.m;
      const int qi = row / p.group;
      const int hq = kvh * p.group + row % p.group;
      const size_t o0 = (static_cast<size_t>(qbase + qi) * p.num_heads + hq) * D + 4 * x.j;
#pragma unroll
      for (int n = 0; n < T::ND; ++n) {
        const f32x4 o = st[r].acc[n] * inv;
        if (p.out_bf16) {
          const uint32_t lo = float_to_bf16_bits(o[0]) | (static_cast<uint32_t>(float_to_bf16_bits(o[1])) << 16);
          const uint32_t hi = float_to_bf16_bits(o[2]) | (static_cast<uint32_t>(float_to_bf16_bits(o[3])) << 16);
          *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p.out) + o0 + 16 * n) = u32x2{lo, hi};
        } else {
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.out) + o0 + 16 * n) = o;
        }
      }
    }
  }
}

__device__ __forceinline__ int xcd_grouped_unit(int id, int NP, int HG);

// bf16: at least two wavefronts per SIMD (two four-wave work-groups per CU).
// With eight or more units per (sequence, kv head), work-groups in index
// order would put a pair's units on every XCD and each XCD's L2 would fetch
// all of its lines; they are grouped onto one XCD instead (xcd_grouped_unit;
// measured on 512-token chunks, 70B-shaped heads, 32 units per pair: 323.2 ->
// 314.7 us; grouping the 4 units per pair of 13B-shaped heads too measured
// 239.5 -> 241.7 us, so those keep index order).  Only the unit -> work-group assignment moves: same results.
template <int KV, int D, int BS, int NW, int RW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(KV == kBf16 ? 2 : 1)))
void decode_wide_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int HX = p.num_kv_heads * p.head_groups;
  const int u = p.head_groups >= 8
                    ? xcd_grouped_unit(static_cast<int>(blockIdx.x), p.num_seqs * p.num_kv_heads, p.head_groups)
                    : static_cast<int>(blockIdx.x);
  run_wide_unit<KV, D, BS, NW, RW>(p, reinterpret_cast<int32_t *>(smem), u / HX, u % HX);
}

// Several units per (sequence, kv head) (more query-head groups than one
// unit holds) read the same K/V.  The hardware deals work-groups to the eight
// XCDs round robin (index mod 8), each XCD with its own L2, so units with
// neighbouring indices would fetch those lines from HBM once per XCD.  Work-
// group index id takes unit (pair, g), pair = sequence * kv_heads + kv head,
// g < HG, laid out in blocks of 8 pairs x HG: the HG units of a pair get
// indices 8 apart, one XCD, and run side by side, so all but the first read
// of a line hit that XCD's L2.  A bijection on [0, NP * HG); returns the
// unit index pair * HG + g.
__device__ __forceinline__ int xcd_grouped_unit(int id, int NP, int HG) {
  const int blk = id / (8 * HG);
  const int in = id - blk * 8 * HG;
  const int nb = min(8, NP - blk * 8);  // pairs in this block (the last may hold fewer)
  return (blk * 8 + in % nb) * HG + in / nb;
}

// ---- units with two row groups per wavefront (MQA-like groups, short causal
// row sets such as a few draft tokens) ------------------------------------------
// Every wavefront holds both row groups of the unit and takes every NW-th
// chunk of the tokens, so each K/V fragment it loads (and, int8 / int4,
// converts) feeds both groups' products.  With the groups on separate
// wavefronts (R = 2 units) every fragment was loaded and converted twice; the
// int8 MQA-like decode was bound by those conversions.  The states are merged
// through LDS one row group at a time.  Causal rows (query token r / G of the
// sequence's nq new tokens, head r % G) mask per lane; chunks that end before
// the unit's first row's position need no mask.  Eight wavefronts per unit,
// one work-group per CU: head_dim 128 with block size 16 takes 225 / 234
// (bf16, single token / causal rows) and 221 / 238 (int4) VGPRs, no spills;
// int8 takes 248-253 and serves single tokens only (with causal rows it
// spills 12-76 bytes per lane).

// QK of both row groups off each converted K fragment (converted once).
template <int KV, int D>
__device__ __forceinline__ void qk_rw(Scores<KV, D> (&S)[2], const KBuf<KV, D> &kb, const QOp<KV, D> (&qop)[2]) {
  using T = Tile<KV, D>;
#pragma unroll
  for (int q = 0; q < T::NQ; ++q) {
    S[0].s[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    S[1].s[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < T::NS; ++s) {
      bf16x8 a;
      if constexpr (KV == kInt8) {
        const u32x4 w = kb.k[q][s >> 1];
        a = (s & 1) ? i8x8_to_bf16x8(w[2], w[3]) : i8x8_to_bf16x8(w[0], w[1]);
      } else if constexpr (KV == kInt4) {
        const u32x2 w = kb.k[q][s >> 1];
        a = i4x8_to_bf16x8_biased((s & 1) ? w[1] : w[0]);
      } else {
        a = __builtin_bit_cast(bf16x8, kb.k[q][s]);
      }
      S[0].s[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[0].q[s], S[0].s[q], 0, 0, 0);
      S[1].s[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[1].q[s], S[1].s[q], 0, 0, 0);
    }
  }
}

// PV of both row groups off each converted V fragment (P as pv_update packs it).
template <int KV, int D, bool TAIL>
__device__ __forceinline__ void pv_rw(State<KV, D> (&st)[2], VBuf<KV, D> &vb, const Probs<KV, D> (&P)[2], int tok0,
                                      int t1) {
  using T = Tile<KV, D>;
  constexpr bool LO = KV != kInt4;
  if constexpr (TAIL && !kQuant<KV>) {
    uint32_t keep[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      keep[k] = ((tok0 + 2 * k < t1) ? 0x0000ffffu : 0u) | ((tok0 + 2 * k + 1 < t1) ? 0xffff0000u : 0u);
#pragma unroll
    for (int n = 0; n < T::ND; ++n)
#pragma unroll
      for (int k = 0; k < 4; ++k) vb.v[n][k] &= keep[k];
  }
#pragma unroll
  for (int r = 0; r < T::NR; ++r) {
    bf16x8 phi[2], plo[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = P[g].p[8 * r + (KV == kInt4 ? kEvenFirst[e] : e)];
        const __bf16 h = static_cast<__bf16>(f);
        phi[g][e] = h;
        if constexpr (LO) {
          const __bf16 lo = static_cast<__bf16>(f - static_cast<float>(h));
          plo[g][e] = lo;
        } else if constexpr (KV == kInt4) {
          st[g].vsum += static_cast<float>(h);
        }
      }
    }
#pragma unroll
    for (int n = 0; n < T::ND; ++n) {
      bf16x8 a;
      if constexpr (KV == kInt8) {
        const u32x4 w = vb.v[n];
        a = r ? i8x8_to_bf16x8(w[2], w[3]) : i8x8_to_bf16x8(w[0], w[1]);
      } else if constexpr (KV == kInt4) {
        const u32x2 w = vb.v[n];
        a = i4x8_to_bf16x8_biased(r ? w[1] : w[0]);
      } else {
        a = __builtin_bit_cast(bf16x8, vb.v[n]);
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        st[g].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi[g], st[g].acc[n], 0, 0, 0);
        if constexpr (LO) st[g].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo[g], st[g].acc[n], 0, 0, 0);
      }
    }
  }
}

template <int KV, int D, int BS, bool TAIL, bool REFILL, bool CAUSAL, bool NT>
__device__ __forceinline__ void consume_rw(State<KV, D> (&st)[2], KBuf<KV, D> &kb, VBuf<KV, D> &vb,
                                           const Ctx<KV, D, BS> &x, const QOp<KV, D> (&qop)[2], const int (&t1r)[2],
                                           int cs, int cn, Ids idn, float scale_log2) {
  using T = Tile<KV, D>;
  Scores<KV, D> S[2];
  qk_rw<KV, D>(S, kb, qop);
  if constexpr (REFILL) {
    __builtin_amdgcn_sched_barrier(0);
    issue_k<NT>(kb, x, cn, idn);
    __builtin_amdgcn_sched_barrier(0);
  }
  Probs<KV, D> P[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    softmax<KV, D, TAIL, CAUSAL>(st[r], S[r], vb, P[r], cs + T::TPL * x.j, CAUSAL ? t1r[r] : x.t1, scale_log2,
                                 qop[r].bias);
  pv_rw<KV, D, TAIL>(st, vb, P, cs + T::TPL * x.j, x.t1);
  if constexpr (REFILL) {
    __builtin_amdgcn_sched_barrier(0);
    issue_v<NT>(vb, x, cn, idn);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int KV, int D, int BS, int NW, bool CAUSAL, bool NT>
__device__ __forceinline__ void run_unit_rw(const DecodeParams &p, const Smem &sm, int b, int hx) {
  using T = Tile<KV, D>;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int kvh = hx / p.head_groups;   // p.head_groups: units per kv head here
  const int rg0 = (hx % p.head_groups) * 2;
  // causal multi-query: the rows of sequence b are its nq new tokens x G
  // heads, query rows q_start[b] .. (a unit with no row, or out-of-bounds
  // offsets, is skipped; uniform over the work-group, before any barrier)
  int qb = b, nq = 1;
  if constexpr (CAUSAL) {
    qb = p.q_start[b];
    nq = p.q_start[b + 1] - qb;
  }
  const int nrows = nq * p.group;
  if (CAUSAL && (rg0 * 16 >= nrows || qb < 0 || qb + nq > p.num_queries || nq > p.max_q_len)) return;
  // rows of several query tokens mask per lane (int8 launches here only with
  // one token per sequence: its masking code would spill)
  constexpr bool ROWS = CAUSAL && KV != kInt8;
  const int TW = p.tbl_window;
  const int32_t *table = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq;
  const int Lraw = p.context_lens[b];
  {
    const int n_first = min(TW, p.max_blocks_per_seq);
    for (int i = threadIdx.x; i < n_first; i += NW * 64) sm.tbl[i] = table[i];
  }
  const int L = min(max(Lraw, 0), p.max_blocks_per_seq * BS);
  Ctx<KV, D, BS> x;
  x.m = lane & 15;
  x.j = lane >> 4;
  x.kvh = kvh;
  x.hkv = p.num_kv_heads;
  x.num_blocks_m1 = p.num_blocks - 1;
  x.kpool = static_cast<const typename KvVec<KV>::T *>(p.k_cache);
  x.vpool = static_cast<const typename KvVec<KV>::T *>(p.v_cache);
  x.kscale = reinterpret_cast<const u32x4 *>(p.k_scale);
  x.vscale = reinterpret_cast<const u32x4 *>(p.v_scale);
  x.tbl = sm.tbl;
  // the unit's positions end at its last row's (all of them for one token)
  x.t1 = CAUSAL ? min(L, L - nq + (min(nrows, (rg0 + 2) * 16) - 1) / p.group + 1) : L;
  x.t1_min = L - nq + (rg0 * 16) / p.group + 1;  // the unit's first row sees positions < t1_min
  x.nbv = (x.t1 + BS - 1) / BS;
  x.newpos = -1;
  x.newblk = -1;
  x.newk = 0u;
  x.newv = 0u;
  x.news = 0u;
  x.scr = nullptr;
  QOp<KV, D> qop[2];
  int gc[2];
  int t1r[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int r0 = (rg0 + r) * 16;
    gc[r] = min(16, nrows - r0);  // <= 0: a row group past the last row
    const bool qvalid = x.m < gc[r];
    const int row = r0 + x.m;
    const int qi = CAUSAL ? row / p.group : 0;
    const int hq = kvh * p.group + (CAUSAL ? row % p.group : row);
    t1r[r] = min(L - nq + qi + 1, x.t1);
    const uint16_t *qrow =
        static_cast<const uint16_t *>(p.q) + (static_cast<size_t>(qb + qi) * p.num_heads + hq) * D;
#pragma unroll
    for (int s = 0; s < T::NS; ++s) {
      const int d0 = kQuant<KV> ? (64 * (s >> 1) + 16 * x.j + 8 * (s & 1)) : (32 * s + 8 * x.j);
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (qvalid) v = *reinterpret_cast<const u32x4 *>(qrow + d0);
      qop[r].q[s] = __builtin_bit_cast(bf16x8, v);
    }
    prepare_qop(qop[r]);
  }
  State<KV, D> st[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int n = 0; n < T::ND; ++n) st[r].acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    st[r].m_run = -INFINITY;
    st[r].l_run = 0.f;
    st[r].vsum = 0.f;
  }
  __syncthreads();
  constexpr int STEP = NW * T::CT;
  for (int ws = 0; ws < x.t1; ws += TW * BS) {
    const int we = min(ws + TW * BS, x.t1);
    x.lb0 = ws / BS;
    if (ws != 0) {
      const int nbw = (we + BS - 1) / BS - x.lb0;
      __syncthreads();
      for (int i = threadIdx.x; i < nbw; i += NW * 64) sm.tbl[i] = table[x.lb0 + i];
      __syncthreads();
    }
    const int nch = (we - ws + T::CT - 1) / T::CT;
    const int n = w < nch ? (nch - w + NW - 1) / NW : 0;
    if (n > 0) {
      KBuf<KV, D> kb;
      VBuf<KV, D> vb;
      int cs = ws + w * T::CT;
      const Ids ids = read_ids(x, cs);
      issue_k<NT>(kb, x, cs, ids);
      issue_v<NT>(vb, x, cs, ids);
      for (int k = 0; k + 1 < n; ++k) {
        const int cn = cs + STEP;
        // the unit's earlier rows cannot see all of a chunk past t1_min
        if (ROWS && cs + T::CT > x.t1_min)
          consume_rw<KV, D, BS, true, true, ROWS, NT>(st, kb, vb, x, qop, t1r, cs, cn, read_ids(x, cn), p.scale_log2);
        else
          consume_rw<KV, D, BS, false, true, ROWS, NT>(st, kb, vb, x, qop, t1r, cs, cn, read_ids(x, cn), p.scale_log2);
        cs = cn;
      }
      consume_rw<KV, D, BS, true, false, ROWS, NT>(st, kb, vb, x, qop, t1r, cs, 0, Ids{0, 0}, p.scale_log2);
    }
  }
  // merge the wavefronts' states, one row group at a time (rows = 16)
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    finish_state(st[r]);
    float l = st[r].l_run + __shfl_xor(st[r].l_run, 16);
    l = l + __shfl_xor(l, 32);
    if (r == 1) __syncthreads();  // the first group's readers are done with the slots
    {
      float *arow = sm.acc + (static_cast<size_t>(w) * 16 + x.m) * (D + 4);
#pragma unroll
      for (int n = 0; n < T::ND; ++n) *reinterpret_cast<f32x4 *>(arow + 16 * n + 4 * x.j) = st[r].acc[n];
      if (x.j == 0) {
        sm.m[w * 16 + x.m] = st[r].m_run;
        sm.l[w * 16 + x.m] = l;
      }
    }
    __syncthreads();
    const int rs0 = (rg0 + r) * 16;
    for (int e = threadIdx.x; e < max(gc[r], 0) * D; e += NW * 64) {
      const int gi = e / D;
      const int d = e % D;
      float M = -INFINITY;
#pragma unroll
      for (int t = 0; t < NW; ++t) M = fmaxf(M, sm.m[t * 16 + gi]);
      float o = 0.f;
      if (M != -INFINITY) {
        float lsum = 0.f, osum = 0.f;
#pragma unroll
        for (int t = 0; t < NW; ++t) {
          const float f = fast_exp2(sm.m[t * 16 + gi] - M);
          lsum += f * sm.l[t * 16 + gi];
          osum += f * sm.acc[(static_cast<size_t>(t) * 16 + gi) * (D + 4) + d];
        }
        o = osum / lsum;
      }
      const int rr = rs0 + gi;
      const int qi = CAUSAL ? rr / p.group : 0;
      const size_t row = static_cast<size_t>(qb + qi) * p.num_heads + kvh * p.group + (CAUSAL ? rr % p.group : rr);
      if (p.out_bf16)
        static_cast<uint16_t *>(p.out)[row * D + d] = float_to_bf16_bits(o);
      else
        static_cast<float *>(p.out)[row * D + d] = o;
    }
  }
}

// at least two wavefronts per SIMD (two four-wave work-groups per CU)
template <int KV, int D, int BS, int NW, bool CAUSAL, bool NT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_rw_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Smem sm = carve<D, NW>(smem, p.tbl_window, 16);
  const int HX = p.num_kv_heads * p.head_groups;
  int rest = xcd_grouped_unit(static_cast<int>(blockIdx.x), p.num_seqs * p.num_kv_heads, p.head_groups);
  run_unit_rw<KV, D, BS, NW, CAUSAL, NT>(p, sm, rest / HX, rest % HX);
}


// One work-group per unit: (sequence, kv head x query-head group[, partition]).
// LPT: a single pass over at most kMaxLptSeqs sequences takes the sequences
// longest first.  The hardware hands out work-groups in index order, so the
// last ones dispatched set the tail of the launch; with the longest units
// first the tail is made of the shortest ones.  Every work-group ranks the
// lengths in LDS (ties by index) and serves the sequence whose rank is its
// index / (head units); the output is the same for any order.
// FUSED: the grid's last work-groups write the new rows (append_rows) and the
// units splice them in.  SHARED: single-row-group units whose siblings read
// the same K/V (ordinary loads, so the lines stay in the XCD's L2).
template <int KV, int D, int BS, int NW, bool CAUSAL = false, int R = 1, bool FUSED = false, bool SHARED = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(FUSED && KV == kInt4 ? 3 : 1)))
void decode_mfma_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Smem sm = carve<D, NW>(smem, p.tbl_window, p.rows_per_group);
  const int HX = p.num_kv_heads * p.head_groups;
  const int nparts = p.partition_size > 0 ? p.max_num_partitions : 1;
  const int id = blockIdx.x;
  if constexpr (FUSED) {
    const int units = HX * p.num_seqs;
    if (id >= units) {  // an append work-group (uniform)
      append_rows<KV, D, BS, NW>(p, id - units, static_cast<int>(gridDim.x) - units);
      return;
    }
  }
  const int part = id / (HX * p.num_seqs);
  int rest = id % (HX * p.num_seqs);
  if (p.partition_size == 0 && p.head_groups > 1)
    rest = xcd_grouped_unit(rest, p.num_seqs * p.num_kv_heads, p.head_groups);
  int b = rest / HX;
  if (p.lpt) {
    constexpr int NT = NW * 64;
    const int B = p.num_seqs;
    const int Lmax = p.max_blocks_per_seq * BS;
    int32_t *len = sm.first;  // len[0..B) lengths, len[B] the chosen sequence
    for (int i = threadIdx.x; i < B; i += NT) len[i] = min(max(p.context_lens[i], 0), Lmax);
    __syncthreads();
    // rank of sequence i = number of sequences ahead of it; `parts` adjacent
    // lanes share one i, each counting a slice of the others, and every
    // thread runs the same number of passes (the shuffles need whole groups)
    int parts = 1;
    while (parts < 16 && parts * 2 * B <= NT) parts *= 2;
    const int slice = threadIdx.x % parts;
    const int per = (B + parts - 1) / parts;
    const int groups = NT / parts;
    const int passes = (B + groups - 1) / groups;
    for (int k = 0; k < passes; ++k) {
      const int i0 = k * groups + static_cast<int>(threadIdx.x) / parts;
      const int i = min(i0, B - 1);
      const int li = len[i];
      const int j1 = min((slice + 1) * per, B);
      int r = 0;
#pragma unroll 8
      for (int j = slice * per; j < j1; ++j) {
        const int lj = len[j];
        r += (lj > li) | ((lj == li) & (j < i));
      }
      for (int off = 1; off < parts; off <<= 1) r += __shfl_xor(r, off);
      if (i0 < B && slice == 0 && r == b) len[B] = i;  // exactly one sequence has rank b
    }
    __syncthreads();
    b = len[B];
  }
  run_unit<KV, D, BS, NW, CAUSAL, R, FUSED, SHARED>(p, sm, b, rest % HX, min(part, nparts - 1));
}

// KV-split pass as a persistent kernel: the grid is sized to the work-groups
// the GPU holds at once, and work-group g takes pieces g, g + grid, ... of the
// non-empty (sequence, kv head x query-head group, partition) pieces only, in
// sequence order.  Each work-group first counts the pieces of every sequence
// (ceil(L / partition_size) x head units) and prefix-sums the counts in LDS;
// a piece index then maps to its sequence by binary search.  No work-group is
// spent on a partition past the end of its sequence, and the pieces are of
// near-equal size, so a static stride balances the work.
template <int KV, int D, int BS, int NW, int R = 1, bool FUSED = false>
__global__ __launch_bounds__(NW * 64) void decode_split_persistent_kernel(DecodeParams p) {
  static_assert(!FUSED || (R == 1 && KV != kInt4), "fused split pieces: bf16 or int8, one unit per piece");
  extern __shared__ __align__(16) unsigned char smem[];
  const Smem sm = carve<D, NW>(smem, p.tbl_window, p.rows_per_group);
  const int HX = p.num_kv_heads * p.head_groups;
  const int B = p.num_seqs;
  const int Lmax = p.max_blocks_per_seq * BS;
  constexpr int NT = NW * 64;

  // pieces of sequence i: first[i] .. first[i + 1] - 1 (exclusive scan of counts)
  const int per = (B + NT - 1) / NT;  // sequences per thread, contiguous
  const int i0 = min(static_cast<int>(threadIdx.x) * per, B);
  const int i1 = min(i0 + per, B);
  int run = 0;
  for (int i = i0; i < i1; ++i) {
    const int L = min(max(p.context_lens[i], 0), Lmax);
    const int c = (L + p.partition_size - 1) / p.partition_size * HX;
    sm.first[i] = run;
    run += c;
  }
  // exclusive scan of the per-thread totals across the work-group
  __shared__ int32_t wsum[NW];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = incl - run;
  for (int v = 0; v < w; ++v) base += wsum[v];
  int total = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) total += wsum[v];
  for (int i = i0; i < i1; ++i) sm.first[i] += base;
  if (threadIdx.x == 0) sm.first[B] = total;
  __syncthreads();

  for (int piece = blockIdx.x; piece < total; piece += gridDim.x) {
    // sequence: the last i with first[i] <= piece (empty sequences share starts)
    int lo = 0, hi = B;  // first[lo] <= piece < first[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm.first[mid] <= piece)
        lo = mid;
      else
        hi = mid;
    }
    const int local = piece - sm.first[lo];
    const int n_b = (sm.first[lo + 1] - sm.first[lo]) / HX;  // partitions of this sequence (>= 1)
    if (n_b > 0) run_unit<KV, D, BS, NW, false, R, FUSED>(p, sm, lo, local / n_b, local % n_b);
  }
  if constexpr (FUSED) append_rows<KV, D, BS, NW>(p, blockIdx.x, gridDim.x);
}

// Split pass: persistent when the sequences' piece offsets fit in LDS,
// else one work-group per (unit, partition).
template <int KV, int D, int BS, int NW, int R = 1>
hipError_t launch_split(const DecodeParams &p_in, hipStream_t s) {
  DecodeParams p = p_in;
  p.head_groups = (p.head_groups + R - 1) / R;  // units per kv head
  const int rows = p.rows_per_group;
  const bool fused = p.append.slot_mapping != nullptr;
  if constexpr (R != 1 || KV == kInt4) {
    if (fused) return hipErrorInvalidValue;  // no fused split kernel for these
  }
  if (fused && p.num_seqs > kMaxPersistentSeqs) return hipErrorInvalidValue;
  if (p.num_seqs <= kMaxPersistentSeqs) {
    const size_t lds = lds_bytes<D, NW>(p.tbl_window, rows, p.num_seqs + 1);
    auto kern = decode_split_persistent_kernel<KV, D, BS, NW, R>;
    if constexpr (R == 1 && KV != kInt4) {
      if (fused) kern = decode_split_persistent_kernel<KV, D, BS, NW, R, true>;
    }
    int per_cu = 0, dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern), NW * 64, lds);
    if (e != hipSuccess) return e;
    const int64_t most = static_cast<int64_t>(p.num_kv_heads) * p.head_groups * p.num_seqs * p.max_num_partitions;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(static_cast<int64_t>(std::max(per_cu, 1)) * cus, most));
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(NW * 64), lds, s, p);
    return hipGetLastError();
  }
  const int64_t nwg = static_cast<int64_t>(p.num_kv_heads) * p.head_groups * p.num_seqs * p.max_num_partitions;
  const size_t lds = lds_bytes<D, NW>(p.tbl_window, rows, 0);
  hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, NW, false, R>), dim3(static_cast<uint32_t>(nwg)), dim3(NW * 64),
                     lds, s, p);
  return hipGetLastError();
}

// Split pieces of MQA-like groups (more than 16 query heads per kv head) take
// two row groups per unit, as single-token units do.
template <int KV, int D, int BS, int NW>
hipError_t launch_split_rows(const DecodeParams &p, hipStream_t s) {
  if (p.head_groups >= 2) return launch_split<KV, D, BS, NW, 2>(p, s);
  return launch_split<KV, D, BS, NW, 1>(p, s);
}

// Single pass: one work-group per unit.  Longest sequences first when the
// batch is small enough to rank in every work-group and the CU holds more
// than one work-group, so that another one streams while a work-group ranks
// (measured: +3 points for four-wave int8 units; with one eight-wave
// work-group per CU the ranking is dead time and cost 2 points).
template <int KV, int D, int BS, int NW, bool CAUSAL = false, int R = 1, bool SHARED = false>
hipError_t launch_single(const DecodeParams &p_in, hipStream_t s) {
  DecodeParams p = p_in;
  p.lpt = (!CAUSAL && NW <= 4 && p.num_seqs <= kMaxLptSeqs) ? 1 : 0;
  p.head_groups = (p.head_groups + R - 1) / R;  // units per kv head
  const int64_t nwg = static_cast<int64_t>(p.num_kv_heads) * p.head_groups * p.num_seqs;
  const size_t lds = lds_bytes<D, NW>(p.tbl_window, p.rows_per_group, p.lpt ? p.num_seqs + 1 : 0);
  if constexpr (!CAUSAL && R == 1) {
    if (p.append.slot_mapping != nullptr) {  // fused append + decode
      // append work-groups after the units, kAppendRowsPerWave rows per wavefront
      const int64_t rows = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads;
      const int64_t per_wg = static_cast<int64_t>(NW) * kAppendRowsPerWave;
      const int64_t extra = (rows + per_wg - 1) / per_wg;
      if (nwg + extra > INT32_MAX) return hipErrorInvalidValue;
      hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, NW, false, 1, true>),
                         dim3(static_cast<uint32_t>(nwg + extra)), dim3(NW * 64), lds, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, NW, CAUSAL, R, false, SHARED>), dim3(static_cast<uint32_t>(nwg)),
                     dim3(NW * 64), lds, s, p);
  return hipGetLastError();
}

// R = row groups per unit.  More than one row group per (sequence, kv head):
// a multi-query unit, or a single-token unit with more than 16 query heads per
// kv head (MQA-like groups).  Packing the groups of a kv head into one unit
// reads its K/V from HBM once instead of once per group, but splits each
// group's tokens between fewer wavefronts, each holding one chunk in flight.
// Units with several query tokens are compute-heavy: all groups in one unit
// (R up to the wavefront count; 512-token chunks ran 2.5x faster than one
// group per unit), except a few groups per kv head (below two per
// wavefront; bf16 and int4), which go two per unit as single-token units do
// when that fills the GPU.  Single-token units stream: two groups per unit, both held
// by every wavefront of the unit (decode_rw_kernel: each K/V fragment, loaded
// and converted once, feeds both groups' products), or one group per unit
// with the units of a kv head sharing its lines through their XCD's L2 when
// two per unit would leave CUs without a work-group (launch_rows).  The
// choice depends on the launch shape only, so a multi-query launch with one
// token per sequence is the single-token launch.
// Wide multi-query units: RW row groups per wavefront, NW * RW per unit.
constexpr int kWideRowGroups = 2;
// Wavefronts per wide unit.  bf16 wide units take four (two work-groups per
// CU at 252 VGPRs): finer grains for the hardware's dispatch than the
// kernel's eight, with the same work per wavefront, so the same results bit
// for bit (measured on 512-token chunks: 13B-shaped heads 251.1 -> 238.5 us,
// 70B-shaped 325.8 -> 323.2 us).  Whether a launch takes wide units is still
// decided on units of NW * RW row groups (use_wide).
template <int KV, int NW>
constexpr int kWideWaves = KV == kBf16 ? 4 : NW;

template <int KV, int D, int BS, int NW>
hipError_t launch_wide(const DecodeParams &p_in, hipStream_t s) {
  DecodeParams p = p_in;
  constexpr int PER_UNIT = NW * kWideRowGroups;
  p.head_groups = (p.head_groups + PER_UNIT - 1) / PER_UNIT;  // units per kv head
  const int64_t nwg = static_cast<int64_t>(p.num_kv_heads) * p.head_groups * p.num_seqs;
  const size_t lds = static_cast<size_t>(p.tbl_window) * 4;
  hipLaunchKernelGGL((decode_wide_kernel<KV, D, BS, NW, kWideRowGroups>), dim3(static_cast<uint32_t>(nwg)),
                     dim3(NW * 64), lds, s, p);
  return hipGetLastError();
}

// Wide units when there are rows for two groups per wavefront and the wide
// launch still gives every CU a work-group (measured: 512-token chunks
// 1.35-1.4x faster than narrow units; 64 tokens x 8 heads on 64 (sequence,
// kv head) pairs, half the CUs idle, 4 % slower).
template <int KV, int D, int BS, int NW>
bool use_wide(const DecodeParams &p, hipError_t &e) {
  constexpr int PER_UNIT = NW * kWideRowGroups;
  const int rg = p.head_groups;
  e = hipSuccess;
  if (p.max_q_len <= 1 || rg < PER_UNIT) return false;
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return false;
  const int64_t units = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads * ((rg + PER_UNIT - 1) / PER_UNIT);
  return units >= cus;
}

// Two-group units (decode_rw_kernel) with NWR wavefronts each; q.head_groups
// is the number of units per kv head.
template <int KV, int D, int BS, int NWR, bool CAUSAL>
hipError_t launch_rw(const DecodeParams &q, hipStream_t s) {
  // several units per (sequence, kv head) read the same lines, side by side
  // on one XCD: ordinary loads, so that all but the first read hit its L2
  // (64 query heads on one kv head, 128 x 4096 tokens: HBM traffic 1.30x
  // -> 1.02x the cache bytes, 63.0 -> 57.0 us); one unit: non-temporal
  const int64_t nwg = static_cast<int64_t>(q.num_kv_heads) * q.head_groups * q.num_seqs;
  const size_t lds = lds_bytes<D, NWR>(q.tbl_window, 16, 0);
  if (q.head_groups > 1) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(decode_rw_kernel<KV, D, BS, NWR, CAUSAL, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_rw_kernel<KV, D, BS, NWR, CAUSAL, false>), dim3(static_cast<uint32_t>(nwg)),
                       dim3(NWR * 64), lds, s, q);
    return hipGetLastError();
  }
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(decode_rw_kernel<KV, D, BS, NWR, CAUSAL, true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_rw_kernel<KV, D, BS, NWR, CAUSAL, true>), dim3(static_cast<uint32_t>(nwg)),
                     dim3(NWR * 64), lds, s, q);
  return hipGetLastError();
}

template <int KV, int D, int BS, int NW, bool CAUSAL>
hipError_t launch_rows(const DecodeParams &p, hipStream_t s) {
  const int rg = p.head_groups;  // row groups of a (sequence, kv head)
  if constexpr (CAUSAL) {
    hipError_t e;
    const bool wide = use_wide<KV, D, BS, NW>(p, e);
    if (e != hipSuccess) return e;
    if (wide) return launch_wide<KV, D, BS, kWideWaves<KV, NW>>(p, s);
  }
  // a few row groups per kv head (a single token, or causal rows below the
  // wide threshold): two per unit, held by every wavefront, when that gives
  // every CU a work-group (measured on one kv head with 64 query heads,
  // 128 x 4096 tokens: bf16 76.7 -> 63.1 us, int8 63.6 -> 48.4 us against two
  // groups on separate wavefronts; 8 draft tokens x 8 heads per kv head,
  // 32 x 2048 tokens: 75.4 -> 70.2 us against one group per wavefront)
  int cus_rw = 0;
  const bool rw_shape = rg >= 2 && (p.max_q_len <= 1 || (CAUSAL && KV != kInt8 && rg < 2 * NW));
  if (rw_shape) {
    int dev = 0;
    hipError_t e0 = hipGetDevice(&dev);
    if (e0 == hipSuccess) e0 = hipDeviceGetAttribute(&cus_rw, hipDeviceAttributeMultiprocessorCount, dev);
    if (e0 != hipSuccess) return e0;
  }
  if (rw_shape && static_cast<int64_t>(p.num_seqs) * p.num_kv_heads * ((rg + 1) / 2) >= cus_rw) {
    DecodeParams q = p;
    q.head_groups = (rg + 1) / 2;  // units per kv head
    // several query tokens per sequence (draft tokens): four-wavefront units,
    // two work-groups per CU (8 draft tokens x 64/8 heads, 32 x 2048 tokens:
    // 64.4 -> 59.4 us against eight); one token (decode, or a multi-query
    // launch bounded to one token, which stays pa_decode bit for bit): eight
    if (CAUSAL && p.max_q_len > 1) return launch_rw<KV, D, BS, 4, CAUSAL>(q, s);
    return launch_rw<KV, D, BS, 8, CAUSAL>(q, s);
  }
  const int most = p.max_q_len > 1 ? NW : 2;
  // single token (also a multi-query launch bounded to one token, which is
  // pa_decode bit for bit), several row groups per kv head: two per unit
  // unless that leaves work-group slots of the GPU empty; then one per unit,
  // the units of a (sequence, kv head) sharing its lines through the L2
  // (ordinary loads; they sit on one XCD)
  if (p.max_q_len <= 1 && rg >= 2) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const size_t lds = lds_bytes<D, NW>(p.tbl_window, p.rows_per_group,
                                        (!CAUSAL && NW <= 4 && p.num_seqs <= kMaxLptSeqs) ? p.num_seqs + 1 : 0);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void *>(decode_mfma_kernel<KV, D, BS, NW, CAUSAL, 1, false, true>),
          NW * 64, lds);
    if (e != hipSuccess) return e;
    const int64_t pairs = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads;
    if (pairs * ((rg + 1) / 2) < static_cast<int64_t>(std::max(per_cu, 1)) * cus)
      return launch_single<KV, D, BS, NW, CAUSAL, 1, true>(p, s);
  }
  int r = 1;
  while (r < rg && r < most) r *= 2;
  switch (r) {
    case 1: return launch_single<KV, D, BS, NW, CAUSAL, 1>(p, s);
    case 2: return launch_single<KV, D, BS, NW, CAUSAL, 2>(p, s);
    case 4: return launch_single<KV, D, BS, NW, CAUSAL, 4>(p, s);
  }
  return launch_single<KV, D, BS, NW, CAUSAL, (NW >= 8 ? 8 : 4)>(p, s);
}

// Wavefronts per unit.  A single-pass bf16 unit is a whole sequence: eight
// wavefronts stream a long one twice as fast as four, which shortens the
// tail of batches with spread-out lengths (one such work-group per CU at this
// kernel's register use).  Split pieces are short and int8 units hold twice
// the tokens per chunk: there four wavefronts and more work-groups per CU
// measured faster.
template <int KV, int D, int BS>
hipError_t launch_t(const DecodeParams &p, hipStream_t s) {
  const bool causal = p.q_start != nullptr;
  if constexpr (kQuant<KV>) {
    if (p.partition_size > 0) return launch_split_rows<KV, D, BS, 4>(p, s);
    if (causal) return launch_rows<KV, D, BS, 4, true>(p, s);
    return launch_rows<KV, D, BS, 4, false>(p, s);
  } else {
    if (p.partition_size > 0) return launch_split_rows<KV, D, BS, 4>(p, s);
    if (causal) return launch_rows<KV, D, BS, 8, true>(p, s);
    return launch_rows<KV, D, BS, 8, false>(p, s);
  }
}

template <int KV, int D>
hipError_t launch_bs(const DecodeParams &p, int bs, hipStream_t s) {
  switch (bs) {
    case 16: return launch_t<KV, D, 16>(p, s);
    case 32: return launch_t<KV, D, 32>(p, s);
    case 64: return launch_t<KV, D, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int KV>
hipError_t launch_kv(const DecodeParams &p, int head_dim, int block_size, hipStream_t s) {
  if (head_dim == 128) return launch_bs<KV, 128>(p, block_size, s);
  if (head_dim == 64) return launch_bs<KV, 64>(p, block_size, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams &p, pa_dtype kv_dtype, int head_dim, int block_size, hipStream_t s) {
  switch (kv_dtype) {
    case PA_BF16: return launch_kv<kBf16>(p, head_dim, block_size, s);
    case PA_I8: return launch_kv<kInt8>(p, head_dim, block_size, s);
    case PA_I4: return launch_kv<kInt4>(p, head_dim, block_size, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
