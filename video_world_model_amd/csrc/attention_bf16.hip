// Attention over the compressed cache, bf16 activations, for gfx950 (CDNA4).
//
// Method: QuantWM rebuilds each Key as centre + dequantized 2-bit residual +
// U c_hat, the PSAC compensation applied at cache reconstruction ([digest]
// "Flickering after quantization? ...", PSAC paragraph; [review] summary: a
// low-rank correction of the attention logits), and each Value as centre +
// dequantized residual ([digest], QSAC paragraph, QVG scheme).  The logits are
// the Query-Key dot products ([abstract]); the output is their softmax-weighted
// sum of Values.
//
// Design:
//  * 8 waves and 256 queries per workgroup (32 per wave, lane = query), one
//    workgroup per CU.  All 8 waves share the rebuild of each 64-key tile.
//  * Two LDS buffers.  While the waves run the MFMAs of tile j from one buffer,
//    every thread rebuilds its share of tile j+1 into the other from registers
//    that were loaded one tile ahead; the centre indices are loaded two tiles
//    ahead because they address the centre rows.  One barrier per tile.
//  * Rebuild by channel pairs.  A pair of 2-bit codes becomes an exact fp16
//    pair by placing the two fields in the mantissa of 1024.0 and subtracting
//    1024; mixed-precision FMAs then form centre + z + c s in fp32 and round
//    each value to fp16 once (7 VALU ops per pair).  Inside each 16-channel
//    group the channels sit in paired order (position 2j holds channel j,
//    position 2j+1 channel j+8), which is where one shift of a code word puts
//    fields j and j+8; queries, centres and U^T use the same order and the
//    output is written back in channel order.
//  * V~ is stored row-major like K~ and read with ds_read_b64_tr_b16, which
//    gives each lane four consecutive keys of one channel: the A operand of
//    O^T += V~^T P^T, without a transposing store.
//  * PSAC as 16 (r <= 16) or 32 (r <= 32) extra contraction columns:
//    q.(k_hat + U c_hat) = q.k_hat + (U^T q).c_hat, with U^T q computed once
//    per workgroup on the MFMA unit.
//  * Online softmax in base 2 with a lazy running max: it only moves when a
//    tile's maximum exceeds it by more than 8, so probabilities stay below 2^8
//    and most tiles skip the rescaling of the accumulators.
//  * All workgroups of one (head, key range) run on one XCD (workgroups are
//    dealt to the 8 XCDs round-robin), so their cache reads share its L2.
//  * Work is split stream-K over (head, query block, key tile) units; query
//    blocks cut between workgroups leave partial results that a small combine
//    kernel merges by log-sum-exp.
//  * The key axis can run through several parts in one launch (a separate
//    kernel, MULTI): compressed caches of successive calibration epochs, each
//    rebuilt with its own centres and compensated with its own U, then
//    optionally the current chunk's own bf16 keys and values.  A segment runs
//    the same pipelined tile loop once per part it touches, with the part's
//    fields fixed and U^T q formed for it; the softmax state carries over.
#include "qwm_internal.h"

#include <algorithm>
#include <climits>
#include <type_traits>

namespace qwm {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s4_t lds_s4;

constexpr int kWaves = 8;              // waves per workgroup (one workgroup per CU)
constexpr int BN = 64;                 // keys per tile
constexpr int kSlotRows = 32 * kWaves;  // partial-result rows per slot (the queries of a workgroup)
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;           // log2 headroom before the running max moves

// Work decomposition (stream-K).  The work units are (head, query block, key
// tile), tile fastest.  Workgroup w takes units [w U / G, (w+1) U / G); a run
// of units inside one (head, query block) pair is a segment.  A pair cut by a
// workgroup boundary leaves partial results (O normalised by its own sum, and
// lse) in workspace slots: slot 2w for workgroup w's first segment, 2w+1 for
// its last; the combine kernel merges them, one block per pair and row
// block.  Without a workspace, G equals the number of pairs and every
// workgroup takes one whole pair.
struct Grid {
  int n_qb;        // query blocks per head
  int qpb;         // queries per block: a multiple of 32, at most BM
  int heads;
  int ntiles;      // key tiles: the compressed caches', then the local chunk's
  int ntc;         // key tiles of the compressed caches
  long long units; // heads * n_qb * ntiles
  int G;           // workgroups with work
  int per_xcd;     // ceil(G / 8): workgroups w of one XCD take a contiguous run
};

__device__ __forceinline__ h2_t as_h2(uint32_t x) { return __builtin_bit_cast(h2_t, x); }
__device__ __forceinline__ uint32_t as_u32(h2_t x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ _Float16 bf_to_h(uint32_t bits) { return (_Float16)__uint_as_float(bits << 16); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// Position of PSAC column k in the K~ rows (and of U^T q in the Q fragment):
// the MFMA that computes U^T q leaves columns 4hf..4hf+3 and 8+4hf..8+4hf+3 in
// lane half hf (within each 16-column k-step; the map swaps bits 2 and 3, so
// it is its own inverse).
__device__ __forceinline__ int psac_col(int k) { return 8 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3); }

// fp16 pitch of the K~ rows in LDS: d channels, 16 or 32 PSAC columns, 8 pad
template <int D, int NPS>
constexpr int kKRow = D + 8 + 16 * (NPS > 1 ? NPS : 1);

// One pair of rebuilt values, each rounded to fp16 once:
//   (mu.lo + (c.lo s + z), mu.hi + (c.hi s + z))
// c: the exact code pair (fp16), zs: half2 (zero, scale), mu: the centre pair
// (fp16).  fma_pair: v_fma_mix_f32 forms c s + z in fp32 from the fp16 halves
// (the product is exact and the fp32 rounding far below fp16's); round_lo/hi:
// v_fma_mixlo/hi_f16 add the centre and round once into each half.
__device__ __forceinline__ void fma_pair(uint32_t c, uint32_t zs, float& t0, float& t1) {
  asm("v_fma_mix_f32 %0, %1, %2, %2 op_sel:[0,1,0] op_sel_hi:[1,1,1]" : "=v"(t0) : "v"(c), "v"(zs));
  asm("v_fma_mix_f32 %0, %1, %2, %2 op_sel:[1,1,0] op_sel_hi:[1,1,1]" : "=v"(t1) : "v"(c), "v"(zs));
}
__device__ __forceinline__ uint32_t round_lo(uint32_t mu, float t0) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(mu), "v"(t0));
  return r;
}
__device__ __forceinline__ void round_hi(uint32_t& r, uint32_t mu, float t1) {
  asm("v_fma_mixhi_f16 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(r) : "v"(mu), "v"(t1));
}

// 16 values centre + z + code * s of one (token, group) in paired channel
// order.  w: the group's code word (channel i in bits 2i, 2i+1); zs: half2
// (zero, scale); m0, m1: the centre's 16 fp16 values in paired order.  Codes j
// and j+8 of one shift land in the low bits of each half; or-ing them into the
// mantissa of 1024.0 (ulp 1) and subtracting 1024 gives them exactly as fp16.
__device__ __forceinline__ void rebuild16(uint32_t w, uint32_t zs, const uint4& m0, const uint4& m1, uint4& o0,
                                          uint4& o1, uint32_t magic_v, uint32_t mask_s) {
  const h2_t magic = as_h2(0x64006400u);  // (1024, 1024)
  const uint32_t mu[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
  uint32_t c[8], r[8];
  float t0[8], t1[8];
  // in stages over the 8 pairs, so that no instruction waits on the one before
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t x;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(x) : "v"(w >> (2 * j)), "s"(mask_s), "v"(magic_v));
    c[j] = as_u32(as_h2(x) - magic);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) fma_pair(c[j], zs, t0[j], t1[j]);
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = round_lo(mu[j], t0[j]);
#pragma unroll
  for (int j = 0; j < 8; ++j) round_hi(r[j], mu[j], t1[j]);
  o0 = make_uint4(r[0], r[1], r[2], r[3]);
  o1 = make_uint4(r[4], r[5], r[6], r[7]);
}

// Part e of the table.  Constant-offset reads only: a dynamic index into the
// by-value kernel argument would make the compiler copy the whole table to
// scratch memory.
__device__ __forceinline__ CachePart part_at(const PartTable& t, int e) {
  switch (e) {
#define QWM_PART_CASE(E) \
    case E:              \
      return t.part[E];
    QWM_PART_CASE(0) QWM_PART_CASE(1) QWM_PART_CASE(2) QWM_PART_CASE(3)
    QWM_PART_CASE(4) QWM_PART_CASE(5) QWM_PART_CASE(6) QWM_PART_CASE(7)
    QWM_PART_CASE(8) QWM_PART_CASE(9) QWM_PART_CASE(10) QWM_PART_CASE(11)
    QWM_PART_CASE(12) QWM_PART_CASE(13) QWM_PART_CASE(14) QWM_PART_CASE(15)
    QWM_PART_CASE(16) QWM_PART_CASE(17) QWM_PART_CASE(18) QWM_PART_CASE(19)
    QWM_PART_CASE(20) QWM_PART_CASE(21) QWM_PART_CASE(22) QWM_PART_CASE(23)
    QWM_PART_CASE(24) QWM_PART_CASE(25) QWM_PART_CASE(26) QWM_PART_CASE(27)
    QWM_PART_CASE(28) QWM_PART_CASE(29) QWM_PART_CASE(30) QWM_PART_CASE(31)
    QWM_PART_CASE(32) QWM_PART_CASE(33) QWM_PART_CASE(34) QWM_PART_CASE(35)
    QWM_PART_CASE(36) QWM_PART_CASE(37) QWM_PART_CASE(38) QWM_PART_CASE(39)
    QWM_PART_CASE(40) QWM_PART_CASE(41) QWM_PART_CASE(42) QWM_PART_CASE(43)
    QWM_PART_CASE(44) QWM_PART_CASE(45) QWM_PART_CASE(46) QWM_PART_CASE(47)
    QWM_PART_CASE(48) QWM_PART_CASE(49) QWM_PART_CASE(50) QWM_PART_CASE(51)
    QWM_PART_CASE(52) QWM_PART_CASE(53) QWM_PART_CASE(54) QWM_PART_CASE(55)
    QWM_PART_CASE(56) QWM_PART_CASE(57) QWM_PART_CASE(58) QWM_PART_CASE(59)
    QWM_PART_CASE(60) QWM_PART_CASE(61) QWM_PART_CASE(62) QWM_PART_CASE(63)
#undef QWM_PART_CASE
    default:
      return t.part[kMaxParts - 1];
  }
}
static_assert(kMaxParts == 64, "part_at covers 64 parts");

// What a launch of the single-cache kernel produces: softmax attention (the
// product), or, from the same tile rebuild and the same S = Q' K~^T, the
// scaled logits [H][n_q][n_k] or each query's top-1 token (debug and
// measurement exports; these run with one workgroup per whole pair).
enum Export { kAttend = 0, kLogits = 1, kTop1 = 2 };

// One segment: pair (head, query block), key tiles [tb, te).  slot < 0: the
// segment covers the pair's whole key range (final output), else partial.
// MULTI: the key axis runs through the parts of the table (compressed caches,
// then the local chunk).  The segment then runs the pipelined tile loop once
// per part it touches, with that part's fields fixed (the loop restarts at a
// part boundary), and forms U^T q again on entering another epoch.
template <int D, int NPS, int NW, bool MULTI, int EX = kAttend>
__device__ __forceinline__ void attend_segment(const AttnParams& p, const Grid& gr, const PartTable* tp,
                                               _Float16* lds, int pair, int tb, int te, int slot) {
  // tp: read by the multi-part instantiation only (null in the other)
  constexpr int NT = 64 * NW;             // threads per workgroup
  constexpr int NG = D / 16;
  constexpr bool PS = NPS > 0;           // PSAC compensation (r > 0)
  constexpr int NPX = PS ? NPS : 1;
  constexpr int NKS = NG + NPS;           // MFMA k-steps of S (the last NPS: PSAC columns)
  constexpr int KROW = kKRow<D, NPS>;     // fp16 pitch of K~ rows: d channels, 16 NPX PSAC columns, 8 pad
  constexpr int VROW = D + 32;            // fp16 pitch of V~ rows
  constexpr int KT = BN * KROW;
  constexpr int BUF = KT + BN * VROW;
  constexpr int NDB = D / 32;             // 32-row blocks of O^T
  constexpr int ITEMS = BN * NG;          // (key, group) rebuild items per tensor
  constexpr int IPT = 2 * ITEMS / NT;     // items per thread
  constexpr int PPT = BN * 8 * NPX / NT;  // PSAC column pairs per thread
  static_assert(IPT * NT == 2 * ITEMS && IPT >= 1 && IPT <= 4, "rebuild split");
  static_assert(PPT * NT == BN * 8 * NPX && PPT >= 1, "PSAC split");

  const int qb = pair % gr.n_qb;
  const int h = pair / gr.n_qb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int q0 = qb * gr.qpb + wave * 32;
  const bool wave_active = wave * 32 < gr.qpb && q0 < p.n_q;  // wave-uniform
  const int qi = q0 + l32;
  const bool qvalid = wave_active && qi < p.n_q;

  // Fields of the compressed cache the tile loop reads: the call's own cache,
  // or one part of the table.
  struct Fields {
    const void* idx_k;
    const void* idx_v;
    const uint32_t* codes_k;
    const uint32_t* codes_v;
    const uint32_t* params_k;
    const uint32_t* params_v;
    const int8_t* coef;
    const uint16_t* coef_scale;
    const uint16_t* mu_k16;
    const uint16_t* mu_v16;
    const uint16_t* ut16;
  };
  auto fields_of = [&](const CachePart& cp) {
    Fields f;
    f.idx_k = cp.cache + tp->idx_k;
    f.idx_v = cp.cache + tp->idx_v;
    f.codes_k = reinterpret_cast<const uint32_t*>(cp.cache + tp->codes_k);
    f.codes_v = reinterpret_cast<const uint32_t*>(cp.cache + tp->codes_v);
    f.params_k = reinterpret_cast<const uint32_t*>(cp.cache + tp->params_k);
    f.params_v = reinterpret_cast<const uint32_t*>(cp.cache + tp->params_v);
    f.coef = reinterpret_cast<const int8_t*>(cp.cache + tp->coef);
    f.coef_scale = reinterpret_cast<const uint16_t*>(cp.cache + tp->coef_scale);
    f.mu_k16 = reinterpret_cast<const uint16_t*>(cp.calib + tp->mu_k16);
    f.mu_v16 = reinterpret_cast<const uint16_t*>(cp.calib + tp->mu_v16);
    f.ut16 = reinterpret_cast<const uint16_t*>(cp.calib + tp->ut16);
    return f;
  };

  // U^T fragments of one calibration, the A operand of the MFMA that forms
  // U^T q: rows 0..16 NPS - 1 are the directions (U^T has 16 NPS rows per
  // head).  Lanes past them read the last row again; an A row only feeds its
  // own output row, and those rows are not used.  All fragments are loaded
  // before the first MFMA, so they cost one memory latency.
  auto load_ut = [&](const uint16_t* ut16, h8_t(&a)[NG]) {
    if constexpr (PS) {
      const uint16_t* ut = ut16 + ((int64_t)h * 16 * NPS + min(l32, 16 * NPS - 1)) * D + 8 * hf;
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) a[ks] = *reinterpret_cast<const h8_t*>(ut + 16 * ks);
    }
  };
  h8_t uta[NG];
  if constexpr (!MULTI) load_ut(p.ut16, uta);  // in flight with the Query loads

  // ---- Q fragment [q | U^T q] in fp16, paired channel order ----
  h8_t qf[NKS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (int64_t)h * p.q_head_stride +
                           (int64_t)(qvalid ? qi : 0) * p.q_token_stride;
#pragma unroll
    for (int ks = 0; ks < NG; ++ks) {
      uint2 a = make_uint2(0u, 0u), b = make_uint2(0u, 0u);
      if (qvalid) {
        a = *reinterpret_cast<const uint2*>(qrow + 16 * ks + 4 * hf);
        b = *reinterpret_cast<const uint2*>(qrow + 16 * ks + 8 + 4 * hf);
      }
      qf[ks] = h8_t{bf_to_h(a.x & 0xffffu), bf_to_h(b.x & 0xffffu), bf_to_h(a.x >> 16), bf_to_h(b.x >> 16),
                    bf_to_h(a.y & 0xffffu), bf_to_h(b.y & 0xffffu), bf_to_h(a.y >> 16), bf_to_h(b.y >> 16)};
    }
  }
  // U^T q into the PSAC k-steps of the Q fragment: accumulator values
  // 8s..8s+7 (output rows of directions 16s..16s+15) fill PSAC k-step s
  auto form_uq = [&](const h8_t(&a)[NG]) {
    if constexpr (PS) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks], qf[ks], acc, 0, 0, 0);
#pragma unroll
      for (int s2 = 0; s2 < NPS; ++s2)
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[NG + s2][i] = (_Float16)acc[8 * s2 + i];
    }
  };
  if constexpr (!MULTI) form_uq(uta);

  // ---- this thread's rebuild items ----
  bool it_v[IPT];
  int it_key[IPT], it_g[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const int it = tid + u * NT;              // items [0, ITEMS) Keys, [ITEMS, 2 ITEMS) Values
    it_v[u] = (ITEMS % NT == 0) ? (u * NT >= ITEMS) : (it >= ITEMS);
    const int local = it % ITEMS;
    it_key[u] = local / NG;
    it_g[u] = local % NG;
  }
  int pk[PPT], ppos[PPT], pcol[PPT];         // PSAC items: key of the tile, k-slot pair, column pair
#pragma unroll
  for (int v = 0; v < PPT; ++v) {
    const int it = tid + v * NT;
    pk[v] = it / (8 * NPX);
    ppos[v] = 2 * (it % (8 * NPX));
    pcol[v] = 16 * (ppos[v] >> 4) + psac_col(ppos[v] & 15);
  }

  const int64_t hN = (int64_t)h * p.Ncap;
  const int64_t hP = (int64_t)h * p.Pcap;

  // Compressed-cache fields of one tile for this thread's items; they stream
  // from HBM, so they are loaded two tiles ahead of their rebuild.  The centre
  // rows (a small, L2-resident table) are loaded one tile ahead.
  struct Raw {
    uint32_t cw[IPT], zs[IPT];
    int idx[IPT];
    int8_t pc0[PPT], pc1[PPT];
    uint16_t psc[PPT];
  };
  uint4 m0[IPT], m1[IPT];
  const uint32_t magic_v = 0x64006400u;  // kept in a VGPR, the mask in an SGPR (one constant-bus read)
  const uint32_t mask_s = 0x00030003u;

  float m_run = -INFINITY;  // running max, log2 units
  float l_run = 0.f;        // this lane's share of the sum of probabilities
  // top-1 export: this lane's best raw score and its key (its keys arrive in
  // increasing order, so a strict comparison keeps the lowest key of a tie)
  float best = -INFINITY;
  int best_k = 0;
  f32x16 o[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;

  const float sl2 = p.scale_log2;
  const int trow = 4 * hf + ((lane & 15) >> 2);             // transposed read: key row in a 16-key chunk
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // and channel position in a 32-channel block

  // The pipelined loop over nt tiles of one part, from key kbeg of that part;
  // kend ends the keys (masked beyond; loads past it read key kend - 1 again).
  // LOC: the part is the local chunk (bf16 rows converted to fp16 in paired
  // channel order, zero PSAC columns) and F is unused.
  auto tile_loop = [&](const Fields& F, int kbeg, int nt, int kend, auto loc_tag) {
    constexpr bool LOC = decltype(loc_tag)::value;
    auto slot_of = [&](int key) { return hN + min(key, kend - 1); };
    auto load_cache = [&](int t0, Raw& r) {
      if constexpr (!LOC) {
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
          const int key = min(t0 + it_key[u], kend - 1);
          const int64_t slot = hN + key;
          const uint32_t fr = ((uint32_t)key + __umulhi((uint32_t)key, p.divF_lo)) >> p.divF_s;
          const int tt = (int)fr * p.tpf + ((key - (int)fr * p.F) >> p.log2T);
          const int g = it_g[u];
          r.cw[u] = (it_v[u] ? F.codes_v : F.codes_k)[slot * NG + g];
          r.zs[u] = (it_v[u] ? F.params_v : F.params_k)[(hP + tt) * NG + g];
          const void* ib = it_v[u] ? F.idx_v : F.idx_k;
          const int bytes = it_v[u] ? p.idx_v_bytes : p.idx_k_bytes;
          r.idx[u] = bytes == 1 ? (int)static_cast<const uint8_t*>(ib)[slot] : (int)static_cast<const uint16_t*>(ib)[slot];
        }
        if constexpr (PS) {
          // unconditional loads (columns past the rank are masked at the rebuild),
          // so that nothing waits for them before the rebuild
#pragma unroll
          for (int v = 0; v < PPT; ++v) {
            const int64_t slot = slot_of(t0 + pk[v]);
            const int8_t* cf = F.coef + slot * p.r;
            r.pc0[v] = cf[min(pcol[v], p.r - 1)];
            r.pc1[v] = cf[min(pcol[v] + 1, p.r - 1)];
            r.psc[v] = F.coef_scale[slot];
          }
        }
      }
    };
    // centre rows of a prefetched tile (local chunk: the rows themselves, of
    // the tile starting at key t0)
    auto load_mu = [&](const Raw& r, int t0) {
#pragma unroll
      for (int u = 0; u < IPT; ++u) {
        const uint16_t* row;
        if constexpr (LOC) {
          const int kk = min(t0 + it_key[u], kend - 1);
          row = it_v[u] ? static_cast<const uint16_t*>(p.v_loc) + (int64_t)h * p.vl_head_stride +
                              (int64_t)kk * p.vl_token_stride
                        : static_cast<const uint16_t*>(p.k_loc) + (int64_t)h * p.kl_head_stride +
                              (int64_t)kk * p.kl_token_stride;
        } else {
          const int c = min(r.idx[u], (it_v[u] ? p.C_v : p.C_k) - 1);
          row = it_v[u] ? F.mu_v16 + ((int64_t)h * p.C_v + c) * D : F.mu_k16 + ((int64_t)h * p.C_k + c) * D;
        }
        const uint4* m = reinterpret_cast<const uint4*>(row + 16 * it_g[u]);
        m0[u] = m[0];
        m1[u] = m[1];
      }
    };
    auto rebuild = [&](int buf, const Raw& r) {
      _Float16* base = lds + buf * BUF;
#pragma unroll
      for (int u = 0; u < IPT; ++u) {
        uint4 o0, o1;
        if constexpr (LOC) {
          // bf16 channel order -> fp16 pairs (channel j, channel j + 8)
          const uint32_t a[4] = {m0[u].x, m0[u].y, m0[u].z, m0[u].w}, b[4] = {m1[u].x, m1[u].y, m1[u].z, m1[u].w};
          uint32_t w[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const uint32_t x = a[jj >> 1], y = b[jj >> 1];
            const float lo = __uint_as_float((jj & 1) ? (x & 0xffff0000u) : (x << 16));
            const float hi = __uint_as_float((jj & 1) ? (y & 0xffff0000u) : (y << 16));
            w[jj] = as_u32(h2_t{(_Float16)lo, (_Float16)hi});
          }
          o0 = make_uint4(w[0], w[1], w[2], w[3]);
          o1 = make_uint4(w[4], w[5], w[6], w[7]);
        } else {
          rebuild16(r.cw[u], r.zs[u], m0[u], m1[u], o0, o1, magic_v, mask_s);
        }
        _Float16* dst = it_v[u] ? base + KT + it_key[u] * VROW + 16 * it_g[u] : base + it_key[u] * KROW + 16 * it_g[u];
        reinterpret_cast<uint4*>(dst)[0] = o0;
        reinterpret_cast<uint4*>(dst)[1] = o1;
      }
      if constexpr (PS) {
#pragma unroll
        for (int v = 0; v < PPT; ++v) {
          if constexpr (LOC) {
            *reinterpret_cast<uint32_t*>(base + pk[v] * KROW + D + ppos[v]) = 0u;
          } else {
            const float sg = (float)__builtin_bit_cast(_Float16, r.psc[v]);
            const float a = pcol[v] < p.r ? (float)r.pc0[v] : 0.f, b = pcol[v] + 1 < p.r ? (float)r.pc1[v] : 0.f;
            *reinterpret_cast<h2_t*>(base + pk[v] * KROW + D + ppos[v]) = h2_t{(_Float16)(a * sg), (_Float16)(b * sg)};
          }
        }
      }
    };

    Raw ra, rb;  // tiles j+1 and j+2
    const int tend = kend;
    if (nt > 0) {
      load_cache(kbeg, ra);
      load_mu(ra, kbeg);
      rebuild(0, ra);
      load_cache(kbeg + BN, ra);
    }
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
      const int t0 = kbeg + j * BN;
      load_mu(ra, t0 + BN);         // centre rows (local chunk: the rows) of tile j+1
      load_cache(t0 + 2 * BN, rb);  // cache fields of tile j+2
      const _Float16* kt = lds + (j & 1) * BUF;
      const _Float16* vt = kt + KT;
      if (__builtin_amdgcn_readfirstlane(wave_active)) {
        // ---- S^T = K~ Q'^T: lane = query, keys 32mb + 8(i/4) + 4hf + i%4 ----
        f32x16 s[2];
        const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // K~ fragments read four ahead of their MFMA (a rolling window)
        constexpr int NF = 2 * NKS;
        auto frag = [&](int f) {
          const int mb = f / NKS, ks = f % NKS;
          return *reinterpret_cast<const h8_t*>(kt + (32 * mb + l32) * KROW + 16 * ks + 8 * hf);
        };
        h8_t win[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) win[f] = frag(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int mb = f / NKS, ks = f % NKS;
          const h8_t a = win[f & 3];
          if (f + 4 < NF) win[f & 3] = frag(f + 4);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[ks], ks == 0 ? zero16 : s[mb], 0, 0, 0);
        }
        // keep four K~ fragments in flight ahead of the MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * NKS - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (__builtin_amdgcn_readfirstlane(t0 + BN > tend)) {  // last tile of a part (uniform)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (t0 + 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3) >= tend) s[mb][i] = -INFINITY;
        }
        if constexpr (EX != kAttend) {
          // exports: keys 32 mb + 8 (i / 4) + 4 hf + i % 4 of this tile (the
          // mapping of the softmax below), masked past the part's end
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = t0 + 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3);
              if constexpr (EX == kLogits) {
                if (qvalid && key < tend) p.logits[((int64_t)h * p.n_q + qi) * p.n_k + key] = s[mb][i] * p.scale;
              } else {
                if (key < tend && s[mb][i] > best) { best = s[mb][i]; best_k = key; }
              }
            }
          rebuild((j + 1) & 1, ra);
        } else {
          // ---- online softmax, base 2 ----
          float mx = s[0][0];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[mb][i]);
          mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
          if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < NDB; ++b)
#pragma unroll
              for (int i = 0; i < 16; ++i) o[b][i] *= alpha;
            m_run = m_new;
          }
          const float moff = -m_run;
          h8_t pf[4];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              pf[2 * mb + (i >> 3)][i & 7] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[mb][i], sl2, moff));
          // the sum uses the rounded probabilities that enter P V (exact products, fp32 sum)
          const h2_t one = h2_t{(_Float16)1.f, (_Float16)1.f};
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int k = 0; k < 4; ++k) l_run = __builtin_amdgcn_fdot2(h2_t{pf[c][2 * k], pf[c][2 * k + 1]}, one, l_run, false);
          // rebuild of the next tile into the other buffer: independent VALU work
          // for the scheduler to place among the P V MFMAs
          rebuild((j + 1) & 1, ra);
          // ---- O^T += V~^T P^T, V~ fragments read two MFMAs ahead ----
          constexpr int NV = 4 * NDB;
          auto vfrag = [&](int f) {
            const int c = f / NDB, b = f % NDB;
            const _Float16* va = vt + (16 * c + trow) * VROW + 32 * b + tcol;
            const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(va));
            const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(va + 8 * VROW));
            return __builtin_bit_cast(h8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          };
          h8_t vw[2] = {vfrag(0), vfrag(1)};
#pragma unroll
          for (int f = 0; f < NV; ++f) {
            const int c = f / NDB, b = f % NDB;
            const h8_t a = vw[f & 1];
            if (f + 2 < NV) vw[f & 1] = vfrag(f + 2);
            o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[c], o[b], 0, 0, 0);
          }
        }
      } else {
        rebuild((j + 1) & 1, ra);
      }
      ra = rb;
      __syncthreads();
    }
  };

  if constexpr (!MULTI) {
    tile_loop(Fields{p.idx_k, p.idx_v, p.codes_k, p.codes_v, p.params_k, p.params_v, p.coef, p.coef_scale,
                     p.mu_k16, p.mu_v16, p.ut16},
              tb * BN, te - tb, min(p.n_k, te * BN), std::false_type{});
  } else {
    // the parts the segment touches, in order (uniform scalar loop); U^T q is
    // formed for the first compressed part and again at each change of part
    bool uq = false;
    for (int e = 0; e < tp->n_parts; ++e) {
      const CachePart cp = part_at(*tp, e);
      const int pend = e + 1 < tp->n_parts ? part_at(*tp, e + 1).tile0 : tp->local0;
      const int a = max(tb, cp.tile0), b = min(te, pend);
      if (a >= b) continue;
      const Fields f = fields_of(cp);
      load_ut(f.ut16, uta);
      form_uq(uta);
      uq = true;
      tile_loop(f, (a - cp.tile0) * BN, b - a, min(cp.n_k, (b - cp.tile0) * BN), std::false_type{});
    }
    const int a = max(tb, tp->local0);
    if (a < te) {
      // local tiles have zero PSAC columns: the Q fragment's U^T q (any, or
      // zero when no compressed part came first) does not enter the scores
      if (!uq) {
#pragma unroll
        for (int ks = NG; ks < NKS; ++ks)
#pragma unroll
          for (int i = 0; i < 8; ++i) qf[ks][i] = (_Float16)0.f;
      }
      const Fields f = fields_of(part_at(*tp, 0));
      tile_loop(f, (a - tp->local0) * BN, te - a, min(p.n_loc, (te - tp->local0) * BN), std::true_type{});
    }
  }

  if (!wave_active) return;
  if constexpr (EX == kTop1) {
    // the two lane halves hold the same query's two key subsets
    const float ob = __shfl_xor(best, 32);
    const int ok = __shfl_xor(best_k, 32);
    if (ob > best || (ob == best && ok < best_k)) best_k = ok;
    if (qvalid && hf == 0) p.top1[(int64_t)h * p.n_q + qi] = best_k;
  }
  if constexpr (EX != kAttend) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (qvalid && hf == 0) {
    if (slot >= 0)
      p.part_ml[(int64_t)slot * kSlotRows + wave * 32 + l32] = lse;
    else if (p.lse)
      p.lse[(int64_t)h * p.n_q + qi] = lse;
  }
  // The wave's 32 output rows go through its own region of LDS (no wave
  // reads the tile buffers after the loop's last barrier): written from the
  // accumulators, then read back as 16-byte row pieces, so that each global
  // store writes whole rows.  Final output in bf16; partials are O
  // normalised by its own sum in fp16 (2^-11 relative, far below the bf16
  // output's rounding), with the lse in fp32.
  constexpr int EP = D + 8;  // fp16 pitch of a row in LDS
  static_assert(NW * 32 * EP <= 2 * (BN * KROW + BN * VROW), "epilogue rows fit in the tile buffers");
  uint16_t* ew = reinterpret_cast<uint16_t*>(lds) + wave * 32 * EP;
  // o[b][4 i4 + t] is stored position sp + t, sp = 32b + 8 i4 + 4hf: channels
  // ch, ch + 8, ch + 1, ch + 9 with ch = (sp & ~15) + (sp & 15) / 2
  auto put_rows = [&](auto cvt) {
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int sp = 32 * b + 8 * i4 + 4 * hf;
        const int ch = (sp & ~15) + ((sp & 15) >> 1);
        uint16_t* e = ew + l32 * EP + ch;
        *reinterpret_cast<uint32_t*>(e) = cvt(o[b][4 * i4] * inv, o[b][4 * i4 + 2] * inv);
        *reinterpret_cast<uint32_t*>(e + 8) = cvt(o[b][4 * i4 + 1] * inv, o[b][4 * i4 + 3] * inv);
      }
  };
  if (slot < 0)
    put_rows([](float a, float b) { return pack_bf16(a, b); });
  else
    put_rows([](float a, float b) { return as_u32(h2_t{(_Float16)a, (_Float16)b}); });
  // the rows are read back by other lanes of the same wave: LDS serves one
  // wave's accesses in order, so only the compiler needs holding back
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // the lane index taken afresh: reusing the one from before the loop
  // keeps it live through the loop, one more VGPR at the limit
  const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  constexpr int PPR = D / 8;     // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int rr = i * RPI + ln / PPR, pc = ln % PPR;
    const uint4 val = *reinterpret_cast<const uint4*>(ew + rr * EP + 8 * pc);
    const int qr = q0 + rr;
    if (qr < p.n_q) {
      uint16_t* dst = slot < 0 ? static_cast<uint16_t*>(p.out) + (int64_t)h * p.o_head_stride + (int64_t)qr * p.o_token_stride
                               : reinterpret_cast<uint16_t*>(p.part_o) + ((int64_t)slot * kSlotRows + wave * 32 + rr) * D;
      *reinterpret_cast<uint4*>(dst + 8 * pc) = val;
    }
  }
}

// MULTI: the key axis runs through the parts of the table (a separate
// kernel, so the single-cache one carries none of their code or arguments)
template <int D, int NPS, int NW, bool MULTI, int EX = kAttend>
__device__ __forceinline__ void attn_bf16_body(const AttnParams& p, const Grid& gr, const PartTable* tbl) {
  constexpr int BUF = BN * kKRow<D, NPS> + BN * (D + 32);
  __shared__ __align__(16) _Float16 lds[2 * BUF];
  const int bid = blockIdx.x;
  const int w = (bid & 7) * gr.per_xcd + (bid >> 3);
  if (w >= gr.G) return;
  if (gr.ntiles == 0) {  // no keys at all: every pair writes zeros and lse = -inf
    attend_segment<D, NPS, NW, MULTI, EX>(p, gr, tbl, lds, w, 0, 0, -1);
    return;
  }
  const long long u0 = (long long)w * gr.units / gr.G;
  const long long u1 = (long long)(w + 1) * gr.units / gr.G;
  long long u = u0;
  bool first = true;
  while (u < u1) {
    const int pair = (int)(u / gr.ntiles);
    const int tb = (int)(u % gr.ntiles);
    const int te = (int)min<long long>(gr.ntiles, tb + (u1 - u));
    const int slot = (tb == 0 && te == gr.ntiles) ? -1 : (first ? 2 * w : 2 * w + 1);
    attend_segment<D, NPS, NW, MULTI, EX>(p, gr, tbl, lds, pair, tb, te, slot);
    u += te - tb;
    first = false;
    __syncthreads();  // the next segment's first rebuild reuses buffer 0
  }
}

template <int D, int NPS, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_bf16_kernel(AttnParams p, Grid gr) {
  attn_bf16_body<D, NPS, NW, false>(p, gr, nullptr);
}

template <int D, int NPS, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_bf16_multi_kernel(AttnParams p, Grid gr, PartTable tbl) {
  attn_bf16_body<D, NPS, NW, true>(p, gr, &tbl);
}

// The logits / top-1 exports of the single-cache kernel (EX: kLogits, kTop1)
template <int D, int NPS, int NW, int EX>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_bf16_export_kernel(AttnParams p, Grid gr) {
  attn_bf16_body<D, NPS, NW, false, EX>(p, gr, nullptr);
}

// Workgroup w whose units [w U / G, (w + 1) U / G) hold unit x (U >= G).
__device__ __forceinline__ int wg_of(long long x, const Grid& gr) {
  int w = (int)(x * gr.G / gr.units);  // its first unit is at most x
  if (w + 1 < gr.G && (long long)(w + 1) * gr.units / gr.G <= x) ++w;
  return w;
}

// Merges the partial results of a pair cut by workgroup boundaries: block
// (pair, rows kCombineRows<D> blockIdx.y .. of its query block), one thread
// per 8 channels of a row (16-byte loads and stores).  The contributors are
// workgroups wa..wb: wa holds the pair in its last segment (its first, when
// its range starts at the pair), the others in their first.  Online over the
// contributors, four at a time so that their loads are in flight together:
//   o = sum_c exp(lse_c - M) o_c / sum_c exp(lse_c - M), lse = M + log sum.
template <int D>
constexpr int kCombineRows = 256 / (D / 8);  // rows per combine block

template <int D>
__global__ __launch_bounds__(256) void combine_sk_kernel(AttnParams p, Grid gr) {
  constexpr int CPT = 8;        // channels per thread
  constexpr int TPR = D / CPT;  // threads per row
  const int pair = blockIdx.x;
  const long long x0 = (long long)pair * gr.ntiles;
  const int wa = wg_of(x0, gr), wb = wg_of(x0 + gr.ntiles - 1, gr);
  if (wa == wb) return;  // one workgroup took the whole pair and wrote it
  const int qb = pair % gr.n_qb, h = pair / gr.n_qb;
  const int r = blockIdx.y * kCombineRows<D> + (int)threadIdx.x / TPR;
  const int rows = min(gr.qpb, p.n_q - qb * gr.qpb);
  if (r >= rows) return;
  const int d0 = ((int)threadIdx.x % TPR) * CPT;
  const int slot_a = ((long long)wa * gr.units / gr.G >= x0) ? 2 * wa : 2 * wa + 1;
  float M = -INFINITY, tot = 0.f, acc[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) acc[j] = 0.f;
  for (int c0 = wa; c0 <= wb; c0 += 4) {
    float l[4];
    h8_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int w = min(c0 + i, wb);
      const int64_t pb = (int64_t)(w == wa ? slot_a : 2 * w) * kSlotRows + r;
      l[i] = c0 + i <= wb ? p.part_ml[pb] : -INFINITY;
      o[i] = *reinterpret_cast<const h8_t*>(reinterpret_cast<const _Float16*>(p.part_o) + pb * D + d0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mn = fmaxf(M, l[i]);
      if (mn == -INFINITY) continue;
      const float a = __expf(M - mn), b = __expf(l[i] - mn);  // M = -inf: a = 0
      tot = fmaf(tot, a, b);
#pragma unroll
      for (int j = 0; j < CPT; ++j) acc[j] = fmaf(acc[j], a, b * (float)o[i][j]);
      M = mn;
    }
  }
  const int qi = qb * gr.qpb + r;
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  uint16_t* dst = static_cast<uint16_t*>(p.out) + (int64_t)h * p.o_head_stride + (int64_t)qi * p.o_token_stride + d0;
  *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv),
                                              pack_bf16(acc[4] * inv, acc[5] * inv), pack_bf16(acc[6] * inv, acc[7] * inv));
  if (d0 == 0 && p.lse) p.lse[(int64_t)h * p.n_q + qi] = tot > 0.f ? M + __logf(tot) : -INFINITY;
}

template <int D, int NPS>
hipError_t launch_t(const AttnParams& p_in, int heads, hipStream_t stream, const PartTable* parts) {
  // the exports take whole pairs (no partial results, no combine pass)
  const int ex = p_in.logits ? kLogits : (p_in.top1 ? kTop1 : kAttend);
  AttnParams p = p_in;
  if (ex != kAttend) p.part_o = nullptr;
  constexpr int BM = 32 * kWaves;               // queries per workgroup
  const int max_wg = kAttnBf16MaxWorkgroups * 8 / kWaves;  // one CU's worth per 8 waves
  Grid g;
  g.heads = heads;
  g.n_qb = (p.n_q + BM - 1) / BM;
  const int per = (p.n_q + g.n_qb - 1) / g.n_qb;  // balance the query blocks
  g.qpb = (per + 31) / 32 * 32;
  // the multi-part kernel's table: tile0 of each part, then local0
  PartTable tbl{};
  int ntc = (p.n_k + BN - 1) / BN;
  if (parts) {
    tbl = *parts;
    ntc = 0;
    for (int e = 0; e < tbl.n_parts; ++e) {
      tbl.part[e].tile0 = ntc;
      ntc += (tbl.part[e].n_k + BN - 1) / BN;
    }
    tbl.local0 = ntc;
  }
  g.ntc = ntc;
  g.ntiles = ntc + (p.n_loc + BN - 1) / BN;
  const long long pairs = (long long)g.n_qb * heads;
  g.units = pairs * g.ntiles;
  if (g.ntiles == 0 || !p.part_o) {
    g.G = (int)pairs;  // one whole pair per workgroup
  } else if (pairs <= max_wg) {
    // k equal pieces per pair (at least 4 tiles each): workgroup boundaries
    // fall on pair boundaries every k workgroups, one segment per workgroup
    const long long k = std::max<long long>(1, std::min<long long>(max_wg / pairs, g.ntiles / 4));
    g.G = (int)(pairs * k);
  } else {
    g.G = max_wg;  // one workgroup per CU, at most two segments each
  }
  g.per_xcd = (g.G + 7) / 8;
  if (p.ev_begin) {
    const hipError_t er = hipEventRecord(static_cast<hipEvent_t>(p.ev_begin), stream);
    if (er != hipSuccess) return er;
  }
  if (ex == kLogits)
    hipLaunchKernelGGL((attn_bf16_export_kernel<D, NPS, kWaves, kLogits>), dim3(g.per_xcd * 8), dim3(64 * kWaves), 0,
                       stream, p, g);
  else if (ex == kTop1)
    hipLaunchKernelGGL((attn_bf16_export_kernel<D, NPS, kWaves, kTop1>), dim3(g.per_xcd * 8), dim3(64 * kWaves), 0,
                       stream, p, g);
  else if (parts)
    hipLaunchKernelGGL((attn_bf16_multi_kernel<D, NPS, kWaves>), dim3(g.per_xcd * 8), dim3(64 * kWaves), 0, stream, p, g,
                       tbl);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, NPS, kWaves>), dim3(g.per_xcd * 8), dim3(64 * kWaves), 0, stream, p, g);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && p.ev_end) e = hipEventRecord(static_cast<hipEvent_t>(p.ev_end), stream);
  if (e != hipSuccess || ex != kAttend || g.G <= 1 || !p.part_o || g.ntiles == 0) return e;
  hipLaunchKernelGGL((combine_sk_kernel<D>), dim3((unsigned)pairs, (g.qpb + kCombineRows<D> - 1) / kCombineRows<D>),
                     dim3(256), 0, stream, p, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16(const AttnParams& p, int heads, int head_dim, hipStream_t stream,
                                 const PartTable* parts) {
  // PSAC k-steps: none (r = 0), one (r <= 16) or two (r <= 32)
  const int nps = p.r == 0 ? 0 : (p.r <= 16 ? 1 : 2);
  if (head_dim == 128) {
    if (nps == 0) return launch_t<128, 0>(p, heads, stream, parts);
    return nps == 1 ? launch_t<128, 1>(p, heads, stream, parts) : launch_t<128, 2>(p, heads, stream, parts);
  }
  if (nps == 0) return launch_t<64, 0>(p, heads, stream, parts);
  return nps == 1 ? launch_t<64, 1>(p, heads, stream, parts) : launch_t<64, 2>(p, heads, stream, parts);
}

}  // namespace qwm
