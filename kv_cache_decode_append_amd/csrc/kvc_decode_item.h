// Internal: the paged GQA decode work item, shared by the decode kernel and
// the mixed-batch kernel.
//
// Each decode step attends the new query over every key and value stored for its
// sequence (aiwithghost.com "KV cache and continuous batching: 1,000 people ask
// AI", section "What does a KV cache keep?"; daviddominguez.dev "The KV cache
// and prefix caching", section "What prefill stores and decode reads"), reading
// them through the sequence's block table (same page, PagedAttention design),
// with several query heads sharing one K/V head (same page, grouped-query
// attention). The read of the whole cache is what grows with context (same page,
// section "The prompt is paid once, the output is paid every step"), so this
// kernel is HBM-bound: it is built to stream K/V at full bandwidth.
//
// Work decomposition (one work item = NW waves: 4 in the decode kernel, 8 in
// the mixed-batch kernel):
//   item = (partition, kv_head, sequence). A partition is `part_blocks`
//   consecutive 16-token blocks of one sequence. Wave w of the item walks
//   blocks w, w+NW, w+2NW, ... of the partition on its own (no barriers in the
//   main loop), keeping an online-softmax state (m, l, acc) for the G query heads of
//   its kv head, so every K/V tile is read from HBM exactly once per kv head.
//   At the end the NW wave states are merged in LDS; a sequence that spans
//   several partitions writes (m, l, acc) partials that decode_merge_kernel
//   combines with the log-sum-exp rule.
//
// Per block (one contiguous (block, kv-head) tile of 16 x head_dim for K and for V):
//   * K and V tiles arrive through 16-byte non-temporal buffer loads (each tile
//     is read once per step), in a register ring of 2-3 blocks per wave. A
//     buffer descriptor of zero bytes turns the prefetch past the wave's last
//     block into a no-op with no memory traffic.
//   * At head dim 128 (bf16 in the decode kernel, fp8 in both kernels) the
//     block step runs on MFMA: QK and PV are two matrix products in one lane
//     layout, straight from the loaded registers (see the MFMA step below). The
//     other head dims, fp32 and the mixed kernel's bf16 item take the
//     dot-product step:
//   * QK: K goes to a per-wave LDS tile with an XOR swizzle of its 16-byte
//     chunks (conflict-free row reads); lane (h, t) computes the full dot product
//     of query head h with token t's key (bf16: v_dot2_f32_bf16, fp32: FMA), so
//     no cross-lane sum is needed. Scores are in the log2 domain (scale*log2 e).
//   * softmax: max and sum over the 16 tokens of a head are DPP reductions
//     inside a row of 16 lanes (8 lanes x 2 for G = 8).
//   * PV: lane owns one 16-byte chunk of a V row and accumulates all G heads;
//     the accumulator is rescaled only when some head's running max moved.

#pragma once

#include <math.h>

#include <type_traits>

#include "kvc.h"
#include "kvc_device.h"

namespace kvc {

constexpr int kMinPartBlocks = 16;

template <typename T, int D, int G, int NW>
struct DecodeShape {
  static constexpr int MAX_PART = NW * 64;     // blocks per partition: one block id per lane
  static constexpr int EB = ElemBytes<T>::value;
  static constexpr int RB = D * EB;             // bytes of one token row of one head
  static constexpr int NC = RB / 16;            // 16-byte chunks per row
  static constexpr int CE = 16 / EB;            // elements per chunk
  static constexpr int TILE = 16 * RB;          // one (block, kv head) tile, bytes
  static constexpr int QS = 2;                  // lanes sharing one (head, token) dot product
  static constexpr int NCQ = NC / QS;           // query chunks held per lane
  static constexpr int LPH = (G == 8) ? 8 : 16; // QK lanes per query head (one DPP row or half)
  static constexpr int TPS = LPH / QS;          // tokens per QK sub-step
  static constexpr int SPL = 16 / TPS;          // QK sub-steps per block
  static constexpr int TPI = 64 / NC;           // V tokens covered by one wave load
  static constexpr int NI = NC / 4;             // 16-byte loads per lane per tile
  // bf16 PV on v_dot2_f32_bf16: a lane holds NI tokens of the same dims, paired up
  static constexpr bool DOT2_PV = (EB == 2) && (NI >= 2);
  // blocks in flight per wave (register ring)
  // (three where the registers allow: 4-wave items, up to 512 VGPRs per lane;
  // the 8-wave items of the mixed kernel have 256 and keep two)
  static constexpr int PF = (EB == 2 && G <= 4 && D <= 128 && NW == 4) ? 3 : 2;
  static constexpr int KST = NW * TILE;         // K staging, all waves
  static constexpr int RED = NW * TPI * G * D * 4;  // end-of-item reduction
  static constexpr int AREA = KST > RED ? KST : RED;
  static constexpr int SMEM = AREA + NW * 16 * G * 4 + NW * G * 8;
  static_assert(NC >= 4 && NC <= 32, "row of 64..512 bytes");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "G in {1,2,4,8}");
};

// Type the kernels compute in: fp8 codes are converted to bf16 (exactly) and
// then take the bf16 path.
template <typename T>
using ComputeT = std::conditional_t<std::is_same_v<T, fp8_tag>, bf16_tag, T>;

struct DecodeArgs {
  const void* q;
  const void* k_new;  // fused append: [B][hkv][D] new K/V at position ctx-1, or null
  const void* v_new;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* ctx_lens;
  void* out;
  float* ws_o;        // [B*Hq][n_part][D]
  float2* ws_ml;      // [B*Hq][n_part]
  int32_t* err;
  int32_t hkv;
  int32_t n_seqs;     // B
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t part_blocks;
  int32_t n_part;
  float scale_log2;   // softmax scale * log2(e)
  float* ks;          // fp8 caches: row scales [num_blocks][hkv][16] of K and V
  float* vs;
};

// Context length the kernels use: clamped to what the grid and table cover.
// `in_bounds` (optional) says whether the caller's length needed no clamping; a
// clamped row is attended over the clamped length but gets no append, since
// its new token's position lies past what the table or the bound covers.
__device__ __forceinline__ int effective_ctx(const DecodeArgs& a, int b, bool report,
                                             bool* in_bounds = nullptr) {
  int ctx = a.ctx_lens[b];
  const int cap = min(a.max_ctx, a.max_blocks * 16);
  const bool ok = ctx >= 0 && ctx <= cap;
  if (!ok) {
    if (report) flag_error(a.err, KVC_DEVERR_CONTEXT);
    ctx = ctx < 0 ? 0 : cap;
  }
  if (in_bounds) *in_bounds = ok;
  return ctx;
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, size_t idx, float x);
template <>
__device__ __forceinline__ void store_out<float>(void* out, size_t idx, float x) {
  reinterpret_cast<float*>(out)[idx] = x;
}
template <>
__device__ __forceinline__ void store_out<bf16_tag>(void* out, size_t idx, float x) {
  reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_bf16_bits(x);
}

// Dot product of one 16-byte chunk pair, 4 independent partial sums.
template <typename T>
__device__ __forceinline__ void chunk_dot(const u32x4& k, const u32x4& q, float (&s)[4]);
template <>
__device__ __forceinline__ void chunk_dot<bf16_tag>(const u32x4& k, const u32x4& q, float (&s)[4]) {
  s[0] = dot2_bf16(k.x, q.x, s[0]);
  s[1] = dot2_bf16(k.y, q.y, s[1]);
  s[2] = dot2_bf16(k.z, q.z, s[2]);
  s[3] = dot2_bf16(k.w, q.w, s[3]);
}
template <>
__device__ __forceinline__ void chunk_dot<float>(const u32x4& k, const u32x4& q, float (&s)[4]) {
  s[0] = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), s[0]);
  s[1] = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), s[1]);
  s[2] = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), s[2]);
  s[3] = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), s[3]);
}

// Unpack a 16-byte chunk into CE fp32 values.
template <typename T, int CE>
__device__ __forceinline__ void unpack(const u32x4& v, float (&x)[CE]);
template <>
__device__ __forceinline__ void unpack<bf16_tag, 8>(const u32x4& v, float (&x)[8]) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
template <>
__device__ __forceinline__ void unpack<float, 4>(const u32x4& v, float (&x)[4]) {
  x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
  x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
}

// One work item: partition `part` of sequence b for kv head kvh, run by the
// NW waves of the calling workgroup (every thread calls it, tid = its thread
// index; smem holds at least DecodeShape<T, D, G, NW>::SMEM bytes). A
// sequence that fits one partition gets its normalised rows written;
// otherwise the item writes its partial (m, l, acc) for decode_merge_kernel.
// A partition holds at most MAX_PART blocks, unless WHOLE: then the waves walk
// it in ranges of MAX_PART blocks, carrying their softmax state from one range
// to the next (the mixed-batch kernel gives a whole sequence to one item).
// FUSE = false compiles the fused append out (the caller has written the new
// token's K/V already).
template <typename T, int D, int G, int NW, bool WHOLE = false, bool FUSE = true>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int kvh, int b, int part,
                                            uint8_t* smem, int tid = threadIdx.x) {
  using C = ComputeT<T>;
  using S = DecodeShape<C, D, G, NW>;
  constexpr bool F8 = std::is_same_v<T, fp8_tag>;
  constexpr int TILE_MEM = F8 ? 16 * D : S::TILE;   // bytes of one (block, kv head) tile
  // fp8 blocks in flight per wave (half a bf16 block each). Three fit in 256
  // registers at head_dim 128 with G <= 4, but on the C3 step two are faster
  // (514 against 491 steps/s): the wave is not waiting on memory there.
  constexpr int PF = F8 ? (D == 128 && G >= 4 ? 2 : 3) : S::PF;
  const int lane = tid & 63;
  // the wave index is uniform across the wave; saying so keeps every buffer
  // descriptor and loop bound in scalar registers (no per-lane waterfall)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq_all = a.hkv * G;

  // The block ids of this wave's first range, read before the context length
  // is known, so that the two reads overlap instead of following each other:
  // the range starts at part * part_blocks whatever the length, every entry
  // of the table row is safe to read, and the entries past the sequence's
  // blocks are dropped once the length is known. (The mixed kernel's
  // whole-sequence item reads its ranges as it reaches them.)
  int32_t first_ids = -1;
  if constexpr (!WHOLE) {
    const int idx = part * a.part_blocks + w + lane * NW;
    if (idx < a.max_blocks && lane * NW + w < a.part_blocks) first_ids = a.bt[(size_t)b * a.max_blocks + idx];
  }

  bool ctx_ok;
  const int ctx = effective_ctx(a, b, part == 0 && kvh == 0 && tid == 0, &ctx_ok);
  const int nblk = (ctx + 15) >> 4;
  const int n_used = nblk > 0 ? (nblk + a.part_blocks - 1) / a.part_blocks : 1;
  if (part >= n_used) return;
  if (ctx == 0) {
    for (int o = tid; o < G * D; o += NW * 64)
      store_out<C>(a.out, ((size_t)b * hq_all + kvh * G) * D + o, 0.f);
    return;
  }
  const int blk_end = min(part * a.part_blocks + a.part_blocks, nblk);
  int blk0 = part * a.part_blocks;   // first block of the range being walked

  uint8_t* kst = smem + w * S::TILE;
  float* plds = reinterpret_cast<float*>(smem + S::AREA) + w * 16 * G;
  uint16_t* p16 = reinterpret_cast<uint16_t*>(plds);          // bf16 weight pairs (DOT2_PV)
  const uint32_t* p32 = reinterpret_cast<const uint32_t*>(plds);
  float2* ml = reinterpret_cast<float2*>(smem + S::AREA + NW * 16 * G * 4);

  // QK layout: lane -> (head h, token slot tt, half qh of the head dim). The two
  // lanes of a pair (qh = 0, 1) hold the two halves of the query row and add
  // their partial dot products with one DPP step.
  const int h = lane / S::LPH, qh = (lane % S::LPH) % S::QS, tt = (lane % S::LPH) / S::QS;
  const bool active = h < G;
  // QK token of the lane's sub-step sl (the lanes of one sub-step read rows
  // 0 .. TPS-1 of a group apart, which keeps the swizzled K reads
  // conflict-free)
  auto tok = [&](int sl) { return tt + S::TPS * sl; };
  u32x4 qv[S::NCQ];
  {
    const int hq = kvh * G + (active ? h : 0);
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint8_t*>(a.q) + ((size_t)b * hq_all + hq) * S::RB);
#pragma unroll
    for (int c = 0; c < S::NCQ; ++c) qv[c] = qp[qh * S::NCQ + c];
  }

  // fp8 at head dim 128: the block step runs on MFMA.
  // Lane (mn = lane % 16, mg = lane / 16). QK: S[token][head] on
  // v_mfma_f32_16x16x32_bf16, A = the K codes of token mn, B = the query of
  // head mn, at the same eight dims per k-step (any permutation of the head
  // dim taken on both operands gives the same dot product); the four lanes of
  // a token read 64 contiguous bytes of its row per load, dims 16mg .. +15
  // and 64 + 16mg .. +15 (k-steps 0, 1 and 2, 3);
  // lane (mn, mg) ends with the scores of tokens 4mg .. 4mg+3 for head mn.
  // PV: O[head][dim] on v_mfma_f32_16x16x16_bf16, A = the weights in exactly
  // that layout (head mn, tokens 4mg .. 4mg+3), B = the V codes of the same
  // four tokens at one dim, 8mn + dt for product dt, transposed in registers
  // from the lane's own 8-byte loads (tokens 4mg .. 4mg+3, dims 8mn .. +7).
  // No tile passes through LDS, and per block a lane issues about half the
  // vector instructions of the dot-product form.
  constexpr bool MF8 = F8 && D == 128;
  // bf16 at head dim 128 (the standalone kernel; the mixed kernel's
  // whole-sequence item keeps the dot-product step, which is as fast there):
  // the same products, k-step kk on dims 32kk + 8mg .. +7 of token mn (again
  // 64 contiguous bytes per token and load), and V transposed in 16-bit halves
  constexpr bool MB16 = std::is_same_v<T, bf16_tag> && D == 128 && !WHOLE;
  constexpr bool MFP = MF8 || MB16;
  const int mn = lane & 15, mg = lane >> 4;
  bf16x8_t qb[4];
  if constexpr (MFP) {
    const int hq = kvh * G + (mn < G ? mn : 0);
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + ((size_t)b * hq_all + hq) * S::RB;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // k-step kk, lane group mg: dims 32kk + 8mg .. +7 (bf16); fp8 takes
      // dims 16mg + 8kk .. +7 for kk < 2 and 64 + 16mg + 8(kk - 2) .. +7
      const int qb_off = MB16 ? 64 * kk + 16 * mg : (kk < 2 ? 32 * mg + 16 * kk : 128 + 32 * mg + 16 * (kk - 2));
      const u32x4 qw = *reinterpret_cast<const u32x4*>(qrow + qb_off);
      qb[kk] = __builtin_bit_cast(bf16x8_t, mn < G ? qw : u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int32_t* bt_row = a.bt + (size_t)b * a.max_blocks;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.kc);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vc);

  // This wave's blocks of the range and their ids, one per lane (a range has
  // at most NW x 64 blocks): inside the loop they are picked with v_readlane,
  // so no block-table load sits behind the prefetch ring in the in-order load
  // counter.
  int n_my = 0;
  int32_t my_blk = -1;
  auto start_range = [&] {
    const int end = WHOLE ? min(blk0 + S::MAX_PART, blk_end) : blk_end;
    // uniform across the wave (said so: the loop bounds and buffer
    // descriptors that derive from it stay in scalar registers)
    n_my = __builtin_amdgcn_readfirstlane((end - blk0 > w) ? (end - blk0 - w + NW - 1) / NW : 0);
    my_blk = lane < n_my ? (WHOLE ? bt_row[blk0 + w + lane * NW] : first_ids) : -1;
  };
  // the first range's block ids are loaded here, next to the query, so that
  // the loads of the new row below are not behind them in the load counter
  start_range();

  // fp8: tile index (block id * Hkv + kv head) of this wave's i-th block, or -1.
  auto tile_of = [&](int i) -> int64_t {
    int64_t tile = -1;
    if (i < n_my) {
      const int blk = __builtin_amdgcn_readlane(my_blk, i);
      if ((unsigned)blk < (unsigned)a.num_blocks)
        tile = (int64_t)blk * a.hkv + kvh;
      else if (lane == 0)
        flag_error(a.err, KVC_DEVERR_BLOCK_ID);
    }
    return tile;
  };
  // Issue the loads of this wave's i-th block into (kb, vb).
  auto issue = [&](u32x4 (&kb)[S::NI], u32x4 (&vb)[S::NI], int i) {
    size_t off = 0;
    uint32_t bytes = 0;
    if (i < n_my) {
      const int blk = __builtin_amdgcn_readlane(my_blk, i);
      if ((unsigned)blk < (unsigned)a.num_blocks) {
        off = ((size_t)blk * a.hkv + kvh) * S::TILE;
        bytes = S::TILE;
      } else if (lane == 0) {
        flag_error(a.err, KVC_DEVERR_BLOCK_ID);
      }
    }
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int j = 0; j < S::NI; ++j) kb[j] = buffer_load16_stream(rk, (uint32_t)(j * 64 + lane) * 16u);
#pragma unroll
    for (int j = 0; j < S::NI; ++j) vb[j] = buffer_load16_stream(rv, (uint32_t)(j * 64 + lane) * 16u);
  };
  // fp8: the codes of the same (token, 8 values) each bf16 load would hold,
  // 8 bytes per lane, and the row scales of the lane's own QK tokens
  // tok(0) .. tok(SPL - 1), each loaded by the lane itself, so that no lane
  // has to fetch another's scale.
  auto issue8 = [&](u32x2 (&kr)[S::NI], u32x2 (&vr)[S::NI], float (&sk)[S::SPL],
                    float (&sv)[S::SPL], int i) {
    const int64_t tile = tile_of(i);
    const size_t off = tile >= 0 ? (size_t)tile * TILE_MEM : 0;
    const uint32_t bytes = tile >= 0 ? TILE_MEM : 0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + off, bytes);
    const __amdgpu_buffer_rsrc_t rks = make_rsrc(a.ks + (tile >= 0 ? tile * 16 : 0), tile >= 0 ? 64u : 0u);
    const __amdgpu_buffer_rsrc_t rvs = make_rsrc(a.vs + (tile >= 0 ? tile * 16 : 0), tile >= 0 ? 64u : 0u);
#pragma unroll
    for (int j = 0; j < S::NI; ++j)
      kr[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                            rk, (uint32_t)(j * 64 + lane) * 8u, 0, kCachePolicyNonTemporal));
#pragma unroll
    for (int j = 0; j < S::NI; ++j)
      vr[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                            rv, (uint32_t)(j * 64 + lane) * 8u, 0, kCachePolicyNonTemporal));
#pragma unroll
    for (int sl = 0; sl < S::SPL; ++sl) {
      const uint32_t soff = (uint32_t)tok(sl) * 4u;
      sk[sl] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, soff, 0, 0));   // default policy,
      sv[sl] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvs, soff, 0, 0));   // as in the MFMA step
    }
  };

  // fp8 on MFMA: one ring slot (K codes of token mn, dims 32mg .. +31; V codes
  // of tokens 4mg .. 4mg+3, dims 8mn .. +7; the K and V row scales of tokens
  // 4mg .. 4mg+3)
  struct Slot8M { u32x4 k[2]; u32x2 v[4]; f32x4 ks, vs; };
  auto issue8m = [&](Slot8M& sl, int i) {
    const int64_t tile = tile_of(i);
    const size_t off = tile >= 0 ? (size_t)tile * TILE_MEM : 0;
    const uint32_t bytes = tile >= 0 ? TILE_MEM : 0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + off, bytes);
    const __amdgpu_buffer_rsrc_t rks = make_rsrc(a.ks + (tile >= 0 ? tile * 16 : 0), tile >= 0 ? 64u : 0u);
    const __amdgpu_buffer_rsrc_t rvs = make_rsrc(a.vs + (tile >= 0 ? tile * 16 : 0), tile >= 0 ? 64u : 0u);
    // the four lanes of a token read 64 contiguous bytes per load: dims
    // 16mg .. +15 and 64 + 16mg .. +15
    sl.k[0] = buffer_load16_stream(rk, (uint32_t)(mn * D + 16 * mg));
    sl.k[1] = buffer_load16_stream(rk, (uint32_t)(mn * D + 64 + 16 * mg));
    // each row scale right after the codes it scales, in the order the block
    // step consumes them: the in-order load counter then lets the softmax
    // start before the V codes land. The scales take the default cache
    // policy: the kv heads' scale rows of one block sit side by side, and
    // their workgroups (one per XCD) read them close together, so the shared
    // cache serves most of them.
    sl.ks = __builtin_bit_cast(f32x4, buffer_load16(rks, 16u * mg));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sl.v[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                              rv, (uint32_t)((4 * mg + j) * D + 8 * mn), 0,
                                              kCachePolicyNonTemporal));
    sl.vs = __builtin_bit_cast(f32x4, buffer_load16(rvs, 16u * mg));
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 om[8];   // MFMA step: O[head 4mg + i][dim 8mn + dt] of product dt
  if constexpr (MFP) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) om[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float acc[G][S::CE];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < S::CE; ++e) acc[hh][e] = 0.f;

  // Fused append. Every load of a tile gives lane `lane` chunk (lane % NC) of
  // some token, so each lane needs one 16-byte chunk of the new row; it is read
  // here, before the pipelined loop (memory operations inside the loop would
  // make the compiler wait on the whole prefetch ring), substituted in
  // registers when the last block is processed, and stored to the cache after
  // the loop. Only the workgroup whose partition holds the last block does so,
  // and nothing is appended for a row whose length had to be clamped (the
  // clamped position holds a valid cached token).
  const bool fuse = FUSE && ctx_ok && a.k_new != nullptr && part == n_used - 1;
  const int t_new = (ctx - 1) & 15;
  u32x4 k_new_c = u32x4{0u, 0u, 0u, 0u}, v_new_c = u32x4{0u, 0u, 0u, 0u};
  auto load_new = [&] {
    const size_t src = ((size_t)b * a.hkv + kvh) * S::RB + (lane % S::NC) * 16;
    k_new_c = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.k_new) + src);
    v_new_c = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.v_new) + src);
  };
  if (!F8 && fuse) load_new();
  // fp8: the new row's codes (this lane's 8 values) and scales, quantised as
  // kv_append does (the NC lanes of each group hold the whole row). The wave
  // that processes the last block makes them there, just before it, so that
  // nothing of the new row is held in registers through the loop; the MFMA
  // step (few registers) loads the row before its loop and quantises it
  // there, so that no load latency sits between its last two blocks.
  u32x2 k_new_q = u32x2{0u, 0u}, v_new_q = u32x2{0u, 0u};
  float k_new_s = 0.f, v_new_s = 0.f;
  bool has_tail = false;   // fp8: this wave processed the sequence's last block
  auto quantise_loaded = [&] {
    if constexpr (F8) {
      const float ka = group_max<S::NC>(bf16x8_amax(k_new_c));
      const float va = group_max<S::NC>(bf16x8_amax(v_new_c));
      if (ka >= kZeroRowAmax) {
        k_new_q = bf16x8_to_e4m3x8(k_new_c, kE4M3Max / ka);
        k_new_s = ka / kE4M3Max;
      }
      if (va >= kZeroRowAmax) {
        v_new_q = bf16x8_to_e4m3x8(v_new_c, kE4M3Max / va);
        v_new_s = va / kE4M3Max;
      }
    }
  };
  auto quantise_new = [&] {
    load_new();
    quantise_loaded();
  };
  // One block, in three phases: score (its K tile to LDS and the scores of
  // its tokens), weigh (the online-softmax update: running max and sum, the
  // PV weights to LDS, the accumulators rescaled) and accumulate (the PV
  // product). TAIL marks the sequence's last block, the only one that can be
  // partial or hold the appended token; every other block skips the masking
  // and substitution code entirely. fp8 passes the row scales of the lane's
  // QK tokens (ks for the scores, vs for the weights) and its V codes.
  auto score = [&](auto tail_tag, u32x4 (&kb)[S::NI], int i, const float (&ks)[S::SPL],
                   float (&s)[S::SPL]) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int lb = blk0 + w + i * NW;
    if constexpr (TAIL && !F8) {
#pragma unroll
      for (int j = 0; j < S::NI; ++j)
        if (fuse && (j * 64 + lane) / S::NC == t_new) kb[j] = k_new_c;
    }
    // K tile -> LDS, chunk c of token t at chunk slot c ^ (t % NC)
#pragma unroll
    for (int j = 0; j < S::NI; ++j) {
      const int ci = j * 64 + lane, tk = ci / S::NC, c = ci % S::NC;
      *reinterpret_cast<u32x4*>(kst + tk * S::RB + ((c ^ (tk % S::NC)) << 4)) = kb[j];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int sl = 0; sl < S::SPL; ++sl) {
      const int t = tok(sl);
      float part_s[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F8) {
        // all of the sub-step's K reads first: the fp8 wave is short of
        // independent work to cover LDS latency (the bf16 wave is not, and
        // keeps the registers)
        u32x4 kk[S::NCQ];
#pragma unroll
        for (int cc = 0; cc < S::NCQ; ++cc) {
          const int c = qh * S::NCQ + cc;
          kk[cc] = *reinterpret_cast<const u32x4*>(kst + t * S::RB + ((c ^ (t % S::NC)) << 4));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cc = 0; cc < S::NCQ; ++cc) chunk_dot<C>(kk[cc], qv[cc], part_s);
      } else {
#pragma unroll
        for (int cc = 0; cc < S::NCQ; ++cc) {
          const int c = qh * S::NCQ + cc;
          const u32x4 kk = *reinterpret_cast<const u32x4*>(kst + t * S::RB + ((c ^ (t % S::NC)) << 4));
          chunk_dot<C>(kk, qv[cc], part_s);
        }
      }
      float dot = (part_s[0] + part_s[1]) + (part_s[2] + part_s[3]);
      dot += dpp_f<kQuadXor1>(dot);                  // the other half of the head dim
      const bool valid = active && (!TAIL || lb * 16 + t < ctx);
      if constexpr (F8) {
        // the key row's scale multiplies its dot product
        s[sl] = valid ? dot * ks[sl] * a.scale_log2 : -INFINITY;
      } else {
        s[sl] = valid ? dot * a.scale_log2 : -INFINITY;
      }
    }
  };

  auto weigh = [&](auto tail_tag, int i, const float (&vs)[S::SPL], const float (&s)[S::SPL]) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int lb = blk0 + w + i * NW;
    // online softmax over this block's tokens, per head (each token sits in
    // both lanes of its pair: harmless for the max, counted once in the sum)
    float mx = s[0];
#pragma unroll
    for (int sl = 1; sl < S::SPL; ++sl) mx = fmaxf(mx, s[sl]);
    mx = group_max<S::LPH>(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_safe);
    float p[S::SPL], ps = 0.f;
#pragma unroll
    for (int sl = 0; sl < S::SPL; ++sl) {
      p[sl] = __builtin_amdgcn_exp2f(s[sl] - m_safe);
      // bf16 PV multiplies by bf16 weights: round once here so that the
      // normaliser l sums exactly the weights the numerator uses. (fp8: the
      // numerator's weight is this rounded p times the value row's scale,
      // rounded to bf16 again below, so there l and the numerator differ by
      // that second rounding, 2^-9 relative at most.)
      if constexpr (S::DOT2_PV) p[sl] = __uint_as_float(f32_to_bf16_bits(p[sl]) << 16);
      ps += (qh == 0) ? p[sl] : 0.f;
    }
    ps = group_sum<S::LPH>(ps);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    float pw[S::SPL];   // the PV weights: p, times the value row's scale for fp8
#pragma unroll
    for (int sl = 0; sl < S::SPL; ++sl) {
      pw[sl] = p[sl];
      if constexpr (F8) {
        // rows past the context may hold NaN scales; their weight is 0
        pw[sl] = (!TAIL || lb * 16 + tok(sl) < ctx) ? p[sl] * vs[sl] : 0.f;
      }
    }
    if (active && qh == 0) {
#pragma unroll
      for (int sl = 0; sl < S::SPL; ++sl) {
        const int t = tok(sl);
        if constexpr (S::DOT2_PV) {
          // packed bf16 pairs in PV order: token t = j*TPI + r sits in pair
          // (j/2)*TPI + r, low half for even j
          const int jt = t / S::TPI, r = t % S::TPI;
          p16[((jt >> 1) * S::TPI + r) * (2 * G) + 2 * h + (jt & 1)] =
              F8 ? (uint16_t)f32_to_bf16_bits(pw[sl]) : (uint16_t)(__float_as_uint(p[sl]) >> 16);
        } else {
          plds[t * G + h] = p[sl];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();

    // rescale the accumulators when a running max moved (rare after the first blocks)
    float al[G];
    bool moved = false;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      al[hh] = readlane_f(alpha, hh * S::LPH);
      moved |= (al[hh] != 1.f);
    }
    if (__builtin_expect(moved, 0)) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < S::CE; ++e) acc[hh][e] *= al[hh];
    }
  };

  // PV: lane owns chunk (lane % NC) of tokens j*TPI + lane / NC, j < NI. vb
  // holds bf16 / fp32 V chunks; v8 the fp8 V codes (8 per lane and load).
  auto accumulate = [&](auto tail_tag, u32x4 (&vb)[S::NI], u32x2 (&v8)[S::NI], int i) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int lb = blk0 + w + i * NW;
    if constexpr (TAIL) {
#pragma unroll
      for (int j = 0; j < S::NI; ++j) {
        const int tk = (j * 64 + lane) / S::NC;
        if (fuse && tk == t_new) {
          if constexpr (F8) v8[j] = v_new_q;
          else vb[j] = v_new_c;
        }
        if (lb * 16 + tk >= ctx) {                                 // unwritten rows may hold NaN
          if constexpr (F8) v8[j] = u32x2{0u, 0u};
          else vb[j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    if constexpr (S::DOT2_PV) {
      // tokens of loads (2m, 2m+1) form a pair; one v_dot2 per (head, dim) and pair
#pragma unroll
      for (int m = 0; m < S::NI / 2; ++m) {
        const int pr = m * S::TPI + lane / S::NC;
        uint32_t pp[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) pp[hh] = p32[pr * G + hh];
        // x[e] = (token a, token b) of dim e as a bf16 pair
        uint32_t x[8];
        if constexpr (F8) {
          // interleave the two tokens' code bytes, then convert pairs: each
          // E4M3 code is a bf16 value, so the pairs equal the bf16 path's
          const u32x2 ca = v8[2 * m], cb = v8[2 * m + 1];
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const uint32_t lo = __builtin_amdgcn_perm(cb[w], ca[w], 0x05010400u);   // a0 b0 a1 b1
            const uint32_t hi = __builtin_amdgcn_perm(cb[w], ca[w], 0x07030602u);   // a2 b2 a3 b3
            x[4 * w + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false));
            x[4 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true));
            x[4 * w + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false));
            x[4 * w + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true));
          }
        } else {
          const u32x4 va = vb[2 * m], vbb = vb[2 * m + 1];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            x[2 * k] = __builtin_amdgcn_perm(vbb[k], va[k], 0x05040100u);
            x[2 * k + 1] = __builtin_amdgcn_perm(vbb[k], va[k], 0x07060302u);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int hh = 0; hh < G; ++hh) acc[hh][e] = dot2_bf16(pp[hh], x[e], acc[hh][e]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < S::NI; ++j) {
        const int tv = j * S::TPI + lane / S::NC;
        float pv[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) pv[hh] = plds[tv * G + hh];
        float x[S::CE];
        unpack<T, S::CE>(vb[j], x);
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
          for (int e = 0; e < S::CE; ++e) acc[hh][e] = fmaf(pv[hh], x[e], acc[hh][e]);
      }
    }
  };

  // bf16 / fp32: the three phases of one block in order.
  auto process = [&](auto tail_tag, u32x4 (&kb)[S::NI], u32x4 (&vb)[S::NI], int i) {
    float s[S::SPL];
    const float none[S::SPL] = {};
    u32x2 no8[S::NI];
    score(tail_tag, kb, i, none, s);
    weigh(tail_tag, i, none, s);
    accumulate(tail_tag, vb, no8, i);
  };

  // fp8: a ring slot's K codes as the bf16 tile the shared path reads, and the
  // row scales of the lane's QK tokens, with the new token's codes and scales
  // in place for the tail block.
  auto k_tile8 = [&](auto tail_tag, const u32x2 (&kr)[S::NI], u32x4 (&kb)[S::NI]) {
    constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
    for (int j = 0; j < S::NI; ++j) {
      u32x2 kx = kr[j];
      if constexpr (TAIL) {
        if (fuse && (j * 64 + lane) / S::NC == t_new) kx = k_new_q;
      }
      kb[j] = e4m3x8_to_bf16x8(kx);
    }
  };
  auto scales8 = [&](auto tail_tag, const float (&sc)[S::SPL], float new_s, float (&out)[S::SPL]) {
    constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
    for (int sl = 0; sl < S::SPL; ++sl) {
      out[sl] = sc[sl];
      if constexpr (TAIL) {
        if (fuse && tok(sl) == t_new) out[sl] = new_s;
      }
    }
  };
  // fp8: the three phases of one block in order.
  auto process8 = [&](auto tail_tag, u32x2 (&kr)[S::NI], u32x2 (&vr)[S::NI],
                      const float (&sk)[S::SPL], const float (&sv)[S::SPL], int i) {
    static_assert(S::DOT2_PV, "fp8 V codes go straight into the packed PV product");
    u32x4 kb[S::NI], vb[S::NI];
    float ks[S::SPL], vs[S::SPL], s[S::SPL];
    k_tile8(tail_tag, kr, kb);
    scales8(tail_tag, sk, k_new_s, ks);
    scales8(tail_tag, sv, v_new_s, vs);
    score(tail_tag, kb, i, ks, s);
    weigh(tail_tag, i, vs, s);
    accumulate(tail_tag, vb, vr, i);
  };

  // fp8 on MFMA: one block. TAIL: the new row's codes and scales in place and
  // rows past the context masked (their codes zeroed: unwritten rows may hold
  // NaN codes, and a zero weight times NaN is NaN in the product).
  auto process8m = [&](auto tail_tag, const Slot8M& sl, int i) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int lb = blk0 + w + i * NW;
    u32x4 kc0 = sl.k[0], kc1 = sl.k[1];
    f32x4 ks = sl.ks, vs = sl.vs;
    u32x2 v8[4] = {sl.v[0], sl.v[1], sl.v[2], sl.v[3]};
    if constexpr (TAIL) {
      if (fuse) {
        // lane c holds the new row's codes of dims 8(c % 16) .. +7; this
        // lane's are chunks 2mg, 2mg + 1, 8 + 2mg, 9 + 2mg
        u32x2 kn[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int src = (c < 2 ? 0 : 8) + 2 * mg + (c & 1);
          kn[c] = u32x2{(uint32_t)__shfl((int)k_new_q.x, src, 64),
                        (uint32_t)__shfl((int)k_new_q.y, src, 64)};
        }
        if (mn == t_new) {
          kc0 = u32x4{kn[0].x, kn[0].y, kn[1].x, kn[1].y};
          kc1 = u32x4{kn[2].x, kn[2].y, kn[3].x, kn[3].y};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * mg + j == t_new) {
            ks[j] = k_new_s;
            vs[j] = v_new_s;
            v8[j] = v_new_q;
          }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lb * 16 + 4 * mg + j >= ctx) v8[j] = u32x2{0u, 0u};
    }
    // QK^T on MFMA: codes to bf16 (exact), four k-steps of 32 dims
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 kw = kk < 2 ? kc0 : kc1;
      const uint32_t d0 = kw[(kk & 1) * 2], d1 = kw[(kk & 1) * 2 + 1];
      const u32x4 kbf = u32x4{
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.f, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.f, true)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.f, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.f, true))};
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kbf), qb[kk], sc, 0, 0, 0);
    }
    // online softmax for head mn over tokens 4mg .. 4mg+3, the max across the
    // four lane groups; the row sum stays per lane until the end. Only the
    // tail block masks: every other block's rows are written, and lanes of
    // heads past G (zero query, so zero scores) hold finite values that are
    // never stored.
    float s[4], mx = -INFINITY;
    float vsm[4] = {vs[0], vs[1], vs[2], vs[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // the key row's scale multiplies its dot product
      s[j] = sc[j] * ks[j] * a.scale_log2;
      if constexpr (TAIL) {
        // rows past the context may hold any bits, their scales too
        const bool valid = mn < G && lb * 16 + 4 * mg + j < ctx;
        s[j] = valid ? s[j] : -INFINITY;
        vsm[j] = valid ? vsm[j] : 0.f;
      }
      mx = fmaxf(mx, s[j]);
    }
    mx = rows_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_safe);
    // the weights rounded to bf16 once, two per conversion (the sum adds
    // them); the PV weights are them times the value rows' scales, rounded
    // again, packed as the products take them
    const uint32_t e01 = pack_bf16x2(__builtin_amdgcn_exp2f(s[0] - m_safe), __builtin_amdgcn_exp2f(s[1] - m_safe));
    const uint32_t e23 = pack_bf16x2(__builtin_amdgcn_exp2f(s[2] - m_safe), __builtin_amdgcn_exp2f(s[3] - m_safe));
    const float p[4] = {bf16_lo(e01), bf16_hi(e01), bf16_lo(e23), bf16_hi(e23)};
    const float ps = ((p[0] + p[1]) + p[2]) + p[3];
    l_run = l_run * alpha + ps;
    m_run = m_new;
    const u32x2 pa = u32x2{pack_bf16x2(p[0] * vsm[0], p[1] * vsm[1]), pack_bf16x2(p[2] * vsm[2], p[3] * vsm[3])};
    // rescale the accumulators when a running max moved: row i of a lane's
    // products is head 4mg + i, whose factor lane 4mg + i holds
    if (__builtin_expect(__ballot(mn < G && alpha != 1.f) != 0, 0)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float al = __shfl(alpha, 4 * mg + j, 64);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) om[dt][j] *= al;
      }
    }
    // PV on MFMA: each 4-byte half of the lane's token rows transposed to
    // (4 tokens) x (one dim) code words, then converted to bf16
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const uint32_t t0 = v8[0][h2], t1 = v8[1][h2], t2 = v8[2][h2], t3 = v8[3][h2];
      const uint32_t lo01 = __builtin_amdgcn_perm(t1, t0, 0x05010400u);   // t0b0 t1b0 t0b1 t1b1
      const uint32_t hi01 = __builtin_amdgcn_perm(t1, t0, 0x07030602u);   // t0b2 t1b2 t0b3 t1b3
      const uint32_t lo23 = __builtin_amdgcn_perm(t3, t2, 0x05010400u);
      const uint32_t hi23 = __builtin_amdgcn_perm(t3, t2, 0x07030602u);
      const uint32_t dd[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),    // dim 4h2 + 0
                              __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),    // dim 4h2 + 1
                              __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),    // dim 4h2 + 2
                              __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};   // dim 4h2 + 3
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32x2 vb = u32x2{
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dd[e], 1.f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dd[e], 1.f, true))};
        om[4 * h2 + e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(s16x4_t, pa), __builtin_bit_cast(s16x4_t, vb), om[4 * h2 + e], 0, 0, 0);
      }
    }
  };

  // bf16 on MFMA: one ring slot (K chunks of token mn, dims 32c + 8mg .. +7
  // for k-step c; V chunks of tokens 4mg .. 4mg+3, dims 8mn .. +7) and one
  // block
  auto issue16m = [&](u32x4 (&kk4)[4], u32x4 (&vv4)[4], int i) {
    size_t off = 0;
    uint32_t bytes = 0;
    if (i < n_my) {
      const int blk = __builtin_amdgcn_readlane(my_blk, i);
      if ((unsigned)blk < (unsigned)a.num_blocks) {
        off = ((size_t)blk * a.hkv + kvh) * S::TILE;
        bytes = S::TILE;
      } else if (lane == 0) {
        flag_error(a.err, KVC_DEVERR_BLOCK_ID);
      }
    }
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int c = 0; c < 4; ++c) kk4[c] = buffer_load16_stream(rk, (uint32_t)(mn * S::RB + 64 * c + 16 * mg));
#pragma unroll
    for (int j = 0; j < 4; ++j) vv4[j] = buffer_load16_stream(rv, (uint32_t)((4 * mg + j) * S::RB + 16 * mn));
  };
  auto process16m = [&](auto tail_tag, const u32x4 (&kk4)[4], const u32x4 (&vv4)[4], int i) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int lb = blk0 + w + i * NW;
    u32x4 kc[4] = {kk4[0], kk4[1], kk4[2], kk4[3]};
    u32x4 vc[4] = {vv4[0], vv4[1], vv4[2], vv4[3]};
    if constexpr (TAIL) {
      if (fuse) {
        // lane c holds the new row's dims 8(c % 16) .. +7; k-step c takes
        // chunk 4c + mg
        u32x4 kn[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) kn[c][e] = (uint32_t)__shfl((int)k_new_c[e], 4 * c + mg, 64);
        if (mn == t_new) {
#pragma unroll
          for (int c = 0; c < 4; ++c) kc[c] = kn[c];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * mg + j == t_new) vc[j] = v_new_c;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lb * 16 + 4 * mg + j >= ctx) vc[j] = u32x4{0u, 0u, 0u, 0u};   // unwritten rows may hold NaN
    }
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kc[kk]), qb[kk], sc, 0, 0, 0);
    // only the tail block masks (see the fp8 step); its rows past the context
    // have zero values, so a zero weight is all they need
    float s[4], mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[j] = sc[j] * a.scale_log2;
      if constexpr (TAIL) s[j] = (mn < G && lb * 16 + 4 * mg + j < ctx) ? s[j] : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    mx = rows_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_safe);
    // bf16 PV multiplies by bf16 weights: round once, two per conversion, and
    // the sum adds the rounded weights; the pairs are the products' operand
    const u32x2 pa = u32x2{
        pack_bf16x2(__builtin_amdgcn_exp2f(s[0] - m_safe), __builtin_amdgcn_exp2f(s[1] - m_safe)),
        pack_bf16x2(__builtin_amdgcn_exp2f(s[2] - m_safe), __builtin_amdgcn_exp2f(s[3] - m_safe))};
    const float ps = ((bf16_lo(pa[0]) + bf16_hi(pa[0])) + bf16_lo(pa[1])) + bf16_hi(pa[1]);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (__builtin_expect(__ballot(mn < G && alpha != 1.f) != 0, 0)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float al = __shfl(alpha, 4 * mg + j, 64);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) om[dt][j] *= al;
      }
    }
    // PV: word e of each token chunk holds dims 8mn + 2e, 2e + 1; pair the
    // four tokens' halves per dim
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
        const u32x2 vb = u32x2{__builtin_amdgcn_perm(vc[1][e], vc[0][e], sel),
                               __builtin_amdgcn_perm(vc[3][e], vc[2][e], sel)};
        om[2 * e + hi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(s16x4_t, pa), __builtin_bit_cast(s16x4_t, vb), om[2 * e + hi], 0, 0, 0);
      }
    }
  };

  // One range of blocks through the ring of PF blocks in flight.
  auto run_range = [&] {
    // Ring of PF blocks in flight; a slot is refilled right after it is used.
    // A wave's blocks ascend, so only its last step can be the sequence's last
    // block: the loop runs the plain path only and the last step is peeled.
    // The loop takes whole turns of the ring only, and the few steps left
    // before the last one follow it: with a step that may be skipped inside
    // the loop, the loop head would have to assume that the refills after it
    // were not made, and its waits for the oldest slot would drain the ring.
    // (The steps after the loop need no refill: every index they would load
    // lies past the wave's blocks.) The mixed kernel's whole-sequence item and
    // G = 8 keep guarded turns: they have no registers to spare for the extra
    // steps (at G = 8 the peeled steps would cost half the waves per SIMD:
    // 5,767 against 4,511 GB/s for bf16 at 64 rows of 2k contexts).
    const int n_main = n_my > 0 ? n_my - 1 : 0;
    if constexpr (MF8) {
      const bool tail_here = fuse && n_my > 0 && blk0 + w + (n_my - 1) * NW == nblk - 1;
      if (tail_here) load_new();
      Slot8M slot[PF];
#pragma unroll
      for (int u = 0; u < PF; ++u) issue8m(slot[u], u);
      if constexpr (WHOLE || G == 8) {
        for (int i = 0; i < n_main; i += PF) {
#pragma unroll
          for (int u = 0; u < PF; ++u) {
            if (i + u < n_main) {
              process8m(std::false_type{}, slot[u], i + u);
              __builtin_amdgcn_sched_barrier(0);
              issue8m(slot[u], i + u + PF);
            }
          }
        }
      } else {
        int i = 0;
        for (; i + PF <= n_main; i += PF) {
#pragma unroll
          for (int u = 0; u < PF; ++u) {
            process8m(std::false_type{}, slot[u], i + u);
            __builtin_amdgcn_sched_barrier(0);
            issue8m(slot[u], i + u + PF);
          }
        }
#pragma unroll
        for (int u = 0; u < PF - 1; ++u)
          if (i + u < n_main) process8m(std::false_type{}, slot[u], i + u);
      }
      if (n_my > 0) {
        const int last = n_my - 1, slot_last = last % PF;
        const bool tail = blk0 + w + last * NW == nblk - 1;
        if (tail_here) {
          quantise_loaded();
          has_tail = true;
        }
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          if (u == slot_last) {
            if (tail)
              process8m(std::true_type{}, slot[u], last);
            else
              process8m(std::false_type{}, slot[u], last);
          }
        }
      }
    } else if constexpr (F8) {
      u32x2 kr[PF][S::NI], vr[PF][S::NI];
      float skr[PF][S::SPL], svr[PF][S::SPL];
#pragma unroll
      for (int u = 0; u < PF; ++u) issue8(kr[u], vr[u], skr[u], svr[u], u);
      if constexpr (WHOLE || G == 8) {
        for (int i = 0; i < n_main; i += PF) {
#pragma unroll
          for (int u = 0; u < PF; ++u) {
            if (i + u < n_main) {
              process8(std::false_type{}, kr[u], vr[u], skr[u], svr[u], i + u);
              __builtin_amdgcn_sched_barrier(0);
              issue8(kr[u], vr[u], skr[u], svr[u], i + u + PF);
            }
          }
        }
      } else {
        int i = 0;
        for (; i + PF <= n_main; i += PF) {
#pragma unroll
          for (int u = 0; u < PF; ++u) {
            process8(std::false_type{}, kr[u], vr[u], skr[u], svr[u], i + u);
            __builtin_amdgcn_sched_barrier(0);
            issue8(kr[u], vr[u], skr[u], svr[u], i + u + PF);
          }
        }
#pragma unroll
        for (int u = 0; u < PF - 1; ++u)
          if (i + u < n_main) process8(std::false_type{}, kr[u], vr[u], skr[u], svr[u], i + u);
      }
      if (n_my > 0) {
        const int last = n_my - 1, slot = last % PF;
        const bool tail = blk0 + w + last * NW == nblk - 1;
        if (tail && fuse) {
          quantise_new();
          has_tail = true;
        }
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          if (u == slot) {
            if (tail)
              process8(std::true_type{}, kr[u], vr[u], skr[u], svr[u], last);
            else
              process8(std::false_type{}, kr[u], vr[u], skr[u], svr[u], last);
          }
        }
      }
    } else if constexpr (MB16) {
      u32x4 k4[S::PF][4], v4[S::PF][4];
#pragma unroll
      for (int u = 0; u < S::PF; ++u) issue16m(k4[u], v4[u], u);
      if constexpr (WHOLE || G == 8) {
        for (int i = 0; i < n_main; i += S::PF) {
#pragma unroll
          for (int u = 0; u < S::PF; ++u) {
            if (i + u < n_main) {
              process16m(std::false_type{}, k4[u], v4[u], i + u);
              __builtin_amdgcn_sched_barrier(0);
              issue16m(k4[u], v4[u], i + u + S::PF);
            }
          }
        }
      } else {
        int i = 0;
        for (; i + S::PF <= n_main; i += S::PF) {
#pragma unroll
          for (int u = 0; u < S::PF; ++u) {
            process16m(std::false_type{}, k4[u], v4[u], i + u);
            __builtin_amdgcn_sched_barrier(0);
            issue16m(k4[u], v4[u], i + u + S::PF);
          }
        }
#pragma unroll
        for (int u = 0; u < S::PF - 1; ++u)
          if (i + u < n_main) process16m(std::false_type{}, k4[u], v4[u], i + u);
      }
      if (n_my > 0) {
        const int last = n_my - 1, slot_last = last % S::PF;
        const bool tail = blk0 + w + last * NW == nblk - 1;
#pragma unroll
        for (int u = 0; u < S::PF; ++u) {
          if (u == slot_last) {
            if (tail)
              process16m(std::true_type{}, k4[u], v4[u], last);
            else
              process16m(std::false_type{}, k4[u], v4[u], last);
          }
        }
      }
    } else {
      u32x4 kb[S::PF][S::NI], vb[S::PF][S::NI];
#pragma unroll
      for (int u = 0; u < S::PF; ++u) issue(kb[u], vb[u], u);
      if constexpr (WHOLE || G == 8) {
        for (int i = 0; i < n_main; i += S::PF) {
#pragma unroll
          for (int u = 0; u < S::PF; ++u) {
            if (i + u < n_main) {
              process(std::false_type{}, kb[u], vb[u], i + u);
              __builtin_amdgcn_sched_barrier(0);
              issue(kb[u], vb[u], i + u + S::PF);
            }
          }
        }
      } else {
        int i = 0;
        for (; i + S::PF <= n_main; i += S::PF) {
#pragma unroll
          for (int u = 0; u < S::PF; ++u) {
            process(std::false_type{}, kb[u], vb[u], i + u);
            // keep the refill of this slot after its use: hoisting the loads
            // above the PV products would force a register copy of the tile
            __builtin_amdgcn_sched_barrier(0);
            issue(kb[u], vb[u], i + u + S::PF);
          }
        }
#pragma unroll
        for (int u = 0; u < S::PF - 1; ++u)
          if (i + u < n_main) process(std::false_type{}, kb[u], vb[u], i + u);
      }
      if (n_my > 0) {
        const int last = n_my - 1, slot = last % S::PF;
        const bool tail = blk0 + w + last * NW == nblk - 1;
#pragma unroll
        for (int u = 0; u < S::PF; ++u) {
          if (u == slot) {
            if (tail)
              process(std::true_type{}, kb[u], vb[u], last);
            else
              process(std::false_type{}, kb[u], vb[u], last);
          }
        }
      }
    }
  };
  run_range();
  if constexpr (WHOLE) {
    for (blk0 += S::MAX_PART; blk0 < blk_end; blk0 += S::MAX_PART) {
      start_range();
      run_range();
    }
  }

  // fused append: write the new token's row (lanes 0..NC-1: K, NC..2NC-1: V;
  // wave 0 for bf16 and fp32, the wave that made the codes for fp8)
  if (fuse && (F8 ? has_tail : w == 0) && lane < 2 * S::NC) {
    const int blk = bt_row[nblk - 1];
    if ((unsigned)blk < (unsigned)a.num_blocks) {
      const size_t prow = ((size_t)blk * a.hkv + kvh) * 16 + t_new;
      uint8_t* base = const_cast<uint8_t*>(lane < S::NC ? kbase : vbase);
      if constexpr (F8) {
        *reinterpret_cast<u32x2*>(base + prow * D + (lane % S::NC) * 8) =
            lane < S::NC ? k_new_q : v_new_q;
        if (lane % S::NC == 0) (lane < S::NC ? a.ks : a.vs)[prow] = lane < S::NC ? k_new_s : v_new_s;
      } else {
        *reinterpret_cast<u32x4*>(base + prow * S::RB + (lane % S::NC) * 16) =
            lane < S::NC ? k_new_c : v_new_c;
      }
    }
  }

  // merge the four wave states
  __syncthreads();
  constexpr int RSUB = MFP ? 1 : S::TPI;          // partial sums per wave, head and dim
  float* red = reinterpret_cast<float*>(smem);   // [NW][RSUB][G][D]
  if constexpr (MFP) {
    l_run = rows_sum(l_run);                     // the four lane groups' partial row sums
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = 4 * mg + j;
      if (hh < G) {
        float* dst = red + (w * G + hh) * D + 8 * mn;
        *reinterpret_cast<f32x4*>(dst) = f32x4{om[0][j], om[1][j], om[2][j], om[3][j]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{om[4][j], om[5][j], om[6][j], om[7][j]};
      }
    }
    if (mg == 0 && mn < G) ml[w * G + mn] = make_float2(m_run, l_run);
  } else {
    const int sub = lane / S::NC, cc = lane % S::NC;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float* dst = red + ((w * S::TPI + sub) * G + hh) * D + cc * S::CE;
#pragma unroll
      for (int e = 0; e < S::CE; e += 4)
        *reinterpret_cast<f32x4*>(dst + e) = f32x4{acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]};
    }
    if (active && lane % S::LPH == 0) ml[w * G + h] = make_float2(m_run, l_run);
  }
  __syncthreads();
  for (int o = tid; o < G * D; o += NW * 64) {
    const int hh = o / D, d = o % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, ml[ww * G + hh].x);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float2 st = ml[ww * G + hh];
      const float f = (st.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.x - M);
      float sum = 0.f;
#pragma unroll
      for (int sub = 0; sub < RSUB; ++sub) sum += red[((ww * RSUB + sub) * G + hh) * D + d];
      L += st.y * f;
      A += sum * f;
    }
    const size_t row = (size_t)b * hq_all + kvh * G + hh;
    if (n_used == 1) {
      store_out<C>(a.out, row * D + d, A / L);
    } else {
      a.ws_o[(row * a.n_part + part) * D + d] = A;
      if (d == 0) a.ws_ml[row * a.n_part + part] = make_float2(M, L);
    }
  }
}

}  // namespace kvc
