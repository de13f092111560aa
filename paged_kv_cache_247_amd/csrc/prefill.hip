// Paged prefill attention with gfx950 matrix cores: each sequence brings Q_i new query tokens
// at positions L_i - Q_i .. L_i - 1, already written to its paged cache, and each token
// attends causally to positions 0 .. its own over the sequence's blocks.
//
// Prefill is the first forward pass over the prompt that fills the cache before generation
// feeds one token at a time (Qualiteg, "About PagedAttention for LLM serving", "Deepening Our
// Understanding of PagedAttention", the past_key_values loop); a chunk of new tokens on top of
// an existing cache is the same computation. The KV cache is reached through the block table
// (same post, "There are logical blocks and physical blocks ..."), as the attention operator
// over non-contiguous KV-cache blocks requires (vAttention, section 3.1).
//
// Work: a workgroup of 4 waves owns (sequence i, kv head g, a tile of 128 / G query tokens):
// 128 rows (token x head of the group, token-major), 32 per wave as two 16-column tiles of
// v_mfma_f32_16x16x32_{bf16,f16}. Unlike decode, the query side is large, so every 32-position
// KV chunk is staged in LDS once per workgroup (buffer loads straight into LDS, spread over the
// waves, a ring of four stages loaded three chunks ahead, one barrier per chunk) and read by
// all four waves: for
// each column tile the logits S^T = K Q^T (rows positions, columns query rows; K rows permuted
// as in decode so that a lane's accumulator holds eight consecutive positions of its own row),
// the causal mask (only on chunks that reach a row's limit) and online softmax of the lane's
// own row, then O^T += V^T P^T with V^T read from LDS as the A operand, and the row sums as a
// tile of ones times P^T. Two workgroups share a CU, so that one's softmax (vector ALU) runs
// beside the other's matrix products instead of in lockstep behind the same barriers.
// Consecutive workgroups take consecutive kv heads, so with 8 kv heads every tile of one head
// runs on the same XCD and the tiles of a sequence share that XCD's L2.
//
// Built with -fno-honor-nans: no arithmetic here meets a NaN (cache slots past a sequence's end
// may hold anything; their logits are replaced by -inf with integer selects and their values
// cleared with bit masks before any arithmetic), so maxima compile to bare v_max3_f32.
#include <type_traits>

#include "prefill.hpp"

namespace pkv {
namespace {

template <Dt DT> struct PMfma;
template <> struct PMfma<Dt::BF16> {
  using V8 = bf16x8;
  static __device__ __forceinline__ f32x4 mac(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ __bf16 narrow(float x) { return (__bf16)x; }
  static constexpr uint32_t kOnePair = 0x3f803f80u;  // two bf16 1.0
};
template <> struct PMfma<Dt::F16> {
  using V8 = f16x8;
  static __device__ __forceinline__ f32x4 mac(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ _Float16 narrow(float x) { return (_Float16)x; }
  static constexpr uint32_t kOnePair = 0x3c003c00u;  // two f16 1.0
};

// At most N vector memory operations of this wave outstanding (they complete in order).
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int kEnc = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kEnc);
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier without memory fences: LDS stages are handed over by the explicit waits
// (each wave's own loads into LDS, each wave's own LDS reads) placed before it.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

constexpr int kBufferFlags = 0x00020000;  // raw buffer descriptor dword 3 (gfx9 family)
constexpr int kStages = 4;                 // LDS stages of KV chunks in flight

template <Dt DT, int D, int S>
__global__ void __launch_bounds__(kPrefillWaves * 64)
prefill_kernel(const PrefillParams a) {
  static_assert(DT == Dt::BF16 || DT == Dt::F16, "16-bit inputs only");
  constexpr int NW = kPrefillWaves;
  constexpr int EB = 2;
  constexpr int CT = 32;             // positions per chunk
  constexpr int BPC = S < CT ? CT / S : 1;  // blocks per chunk
  constexpr int CPK = S > CT ? S / CT : 1;  // chunks per block
  constexpr int CS = S < CT ? S : CT;       // positions of a chunk in one block
  constexpr int KK = D / 32;         // k-steps of the logits product
  constexpr int NT = D / 16;         // 16-row tiles of the output product
  constexpr int RB = D * EB;         // bytes of one K row
  constexpr int NPC = RB / 16;       // sixteen-byte pieces per K row
  constexpr int KB = CT * RB;        // K bytes of a chunk
  constexpr int VB = CT * D * EB;    // V^T bytes of a chunk
  constexpr int STAGE = KB + VB;
  constexpr int TILE = S * D * EB;   // one (block, kv head) tile of K or V^T
  // The part of a block's tile one chunk reads: the whole tile up to 32 positions, else 32 K
  // rows and one 32-position V^T column group (V is stored in groups of min(S, 32)).
  constexpr int CTILE = CS * D * EB;
  constexpr int NLK = KB / 1024;     // 1 KiB loads per chunk: K, then V^T
  constexpr int NLV = VB / 1024;
  constexpr int LPW = (NLK + NLV) / NW;  // loads per wave per chunk
  constexpr int PPT = CTILE / 1024;  // 1 KiB pieces of a chunk's V^T tile
  static_assert((NLK + NLV) % NW == 0 && NLK % LPW == 0, "loads split evenly over the waves");
  static_assert(S % (1024 / RB) == 0 && CTILE % 1024 == 0, "a 1 KiB load stays within one block");
  using M = PMfma<DT>;
  using V8 = typename M::V8;
  using T = typename Elt<DT>::T;
  __shared__ __attribute__((aligned(16))) char smem[kStages * STAGE];

  const int Hkv = a.num_kv_heads;
  const int H = a.num_heads;
  const int G = H / Hkv;
  const int MB = a.max_blocks_per_seq;
  const int w = blockIdx.x;
  const int g = w % Hkv;
  int unit = a.work_items ? a.work_items[w / Hkv] : w / Hkv;
  unit = min(max(unit, 0), a.num_seqs * a.num_tiles - 1);
  const int i = unit / a.num_tiles;
  const int tile = unit % a.num_tiles;
  const int lane = lane_id();
  const int wave = wave_id();
  const int r = lane >> 4;
  const int c = lane & 15;

  const int TQ = kPrefillRows / G;  // query tokens per tile
  const int q0 = a.query_start[i];
  int L = a.context_lens[i];
  L = min(max(L, 0), MB * S);
  const int Q = min(max(a.query_start[i + 1] - q0, 0), L);
  const int tok0 = tile * TQ;
  if (tok0 >= Q) return;  // the whole workgroup: no barrier is pending
  const int ntok = min(TQ, Q - tok0);
  const int base = L - Q + tok0;    // position of the tile's first token
  const int nch = (base + ntok - 1) / CT + 1;
  // This wave's rows: tokens [wt0, wt1] of the tile (clamped to the real ones).
  const int wt0 = (wave * 32) / G;
  const int wt1 = min((wave * 32 + 31) / G, ntok - 1);
  const bool wave_live = wt0 < ntok;

  // Lane (r, c) owns row rr = 32 wave + 16 j + c of each column tile j: token rr / G, head
  // g G + rr % G. Rows past the chunk's tokens compute on zero queries and are not stored.
  // A negative scale is carried by the queries: flipping their sign bits is exact, and then
  // the logits' scale factor cl is positive, so the scaled maximum is cl times the raw one.
  const bool flip = a.scale_log2e < 0.0f;
  const float cl = flip ? -a.scale_log2e : a.scale_log2e;
  int plim[2];
  bool valid[2];
  size_t orow[2];
  V8 qb[2][KK];
  const char* qbase = reinterpret_cast<const char*>(a.q);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rr = wave * 32 + 16 * j + c;
    const int t = rr / G;
    valid[j] = t < ntok;
    const int tt = valid[j] ? t : ntok - 1;
    plim[j] = base + tt;
    orow[j] = ((size_t)(q0 + tok0 + tt) * H + (size_t)g * G + rr % G) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (valid[j]) v = *reinterpret_cast<const u32x4*>(qbase + (orow[j] + 32 * kk + 8 * r) * EB);
      if (flip) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qb[j][kk] = __builtin_bit_cast(V8, v);
    }
  }

  // Block ids: one VGPR holds 64 consecutive logical blocks of the sequence, lane e holding
  // block 64 kb + e; refilled (once per 64 blocks) with one coalesced load that waits for
  // itself. It is issued as an inline instruction: a compiler-visible load here would make
  // the compiler wait for all loads in flight before every later use of the ids. Lanes past
  // the table row read its last entry (ids of blocks past the context are never used).
  const int32_t* bt = a.block_tables + (size_t)i * MB;
  auto load_id_batch = [&](int kb) {
    const int32_t* p = bt + min(64 * kb + lane, MB - 1);
    int v;
    asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)"
                 : "=v"(v) : "v"(p) : "memory");
    return v;
  };
  int id_batch = load_id_batch(0);
  int id_kb = 0;
  auto block_id = [&](int lb) {  // lb: logical block, in the current batch
    const int id = __builtin_amdgcn_readlane(id_batch, lb & 63);
    return min(max(id, 0), a.num_blocks - 1);
  };

  const size_t id_stride = (size_t)Hkv * TILE;
  const char* kpool = reinterpret_cast<const char*>(a.k_cache) + (size_t)g * TILE;
  const char* vpool = reinterpret_cast<const char*>(a.v_cache) + (size_t)g * TILE;
  // ro: bytes from the block's tile to the chunk's part (nonzero only for blocks over 32; K
  // rows and V^T groups of a chunk are the same number of bytes in).
  auto rsrc = [&](const char* pool, int id, int ro) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(pool + (size_t)id * id_stride + ro), 0, TILE - ro, kBufferFlags);
  };
  // Placement of a K row's pieces. A wave's 16-byte LDS read is served in four passes of 16
  // lanes over the 256 bytes of bank space (gfx950: lanes 0-7 with 24-31, 8-15 with 16-23,
  // and the same in the upper half, as the bank-conflict counter shows for test patterns), so
  // a conflict-free read needs each pass's 16 pieces in 16 different 16-byte bank slots. With
  // 256-byte rows (head_dim 128) the slot is the rotated piece index: rows 0-3 and 8-11 (and
  // 4-7, 12-15) must take the eight even rotations and rows 16-19 and 24-27 the same, which
  // 2 (t mod 4) + 8 (t / 8 mod 2) does (lane (r, c) adds r, odd for half of each pass).
  // With 128-byte rows (head_dim 64) two rows share the bank space and t + 4 (t / 16) is
  // conflict-free as it is.
  auto rot = [](int t) {
    return NPC == 16 ? 2 * (t & 3) + 8 * ((t >> 3) & 1) : t + 4 * (t >> 4);
  };

  // This wave's share of chunk n's loads into stage st: LPW consecutive 1 KiB pieces, all of
  // K or all of V^T and all of one block (so one block id and one descriptor per chunk).
  // K pieces are rows of the chunk with their 16-byte parts rotated as in decode; V^T pieces
  // are contiguous 1 KiB of a block's [D][S] tile (of a [D][32] column group past 32).
  static_assert(CTILE % (LPW * 1024) == 0, "a wave's loads of a chunk stay within one block");
  const int x0 = wave * LPW;  // first piece: K pieces 0 .. NLK - 1, then V^T pieces
  const bool wave_k = x0 < NLK;
  const int xb = wave_k ? x0 : x0 - NLK;
  const int wave_blk = xb * 1024 / CTILE;  // block of the chunk these pieces come from
  auto issue = [&](int n, int st) {
    const int lb = BPC == 2 ? n * BPC + wave_blk : n / CPK;  // logical block
    if (lb >= 64 * (id_kb + 1)) {
      id_kb = lb / 64;
      id_batch = load_id_batch(id_kb);
    }
    char* dst = smem + st * STAGE + (wave_k ? 0 : KB);
    // (A named descriptor: passed as a temporary, the host pass drops the kernel stub.)
    const __amdgpu_buffer_rsrc_t rs =
        rsrc(wave_k ? kpool : vpool, block_id(lb), (n % CPK) * CT * RB);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int x = xb + j;
      int voff;
      if (wave_k) {
        const int t = x * (1024 / RB) + lane / NPC;
        voff = (t % S) * RB + ((lane % NPC - rot(t)) & (NPC - 1)) * 16;
      } else {
        voff = (x % PPT) * 1024 + lane * 16;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + x * 1024), 16, voff, 0, 0, 0);
    }
  };

  // Operand reads from a stage (explicit LDS reads; the caller's barrier made the stage whole).
  // K is read first and waited for here; the V^T reads stay in flight behind the logits and
  // the softmax until wait_v (LDS reads complete in order).
  const int k_tau = 8 * (c >> 2) + (c & 3);
  auto read_stage = [&](int st, u32x4 (&kr)[2][KK], u32x4 (&vr)[NT]) {
    const char* ks = smem + st * STAGE;
    const char* vs = ks + KB;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int t = k_tau + 4 * gi;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(
            ks + t * RB + ((4 * kk + r + rot(t)) & (NPC - 1)) * 16);
        asm volatile("ds_read_b128 %0, %1" : "=v"(kr[gi][kk]) : "v"(addr) : "memory");
      }
    }
    // V^T rows d = 16 nt + c: the nt step is a constant, carried in the instruction's offset.
    const char* vp = (S == 16) ? vs + (r >> 1) * TILE + c * (S * EB) + (r & 1) * 16
                               : vs + c * (CS * EB) + r * 16;
    const uint32_t vaddr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)vp;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      asm volatile("ds_read_b128 %0, %1 offset:%2"
                   : "=v"(vr[nt]) : "v"(vaddr), "i"(16 * nt * CS * EB) : "memory");
    static_assert(NT <= 15, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" :: "i"(NT) : "memory");
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(kr[gi][kk]));
  };
  auto wait_v = [&](u32x4 (&vr)[NT]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(vr[nt]));
  };

  // Online softmax with a lazily moved reference: m[j] is the row's reference maximum (log2
  // units), lsum[j] the row's sum of 2^(s - m) (every element of it: the sum comes from the
  // matrix cores, a tile of ones times P^T, so it adds exactly the 16-bit weights that multiply
  // V). A chunk whose maximum stays within kSlack of the reference uses it as it is: its
  // weights are at most 2^kSlack, which the 16-bit P operand and the fp32 sums hold as well as
  // weights below 1. Only when a row's maximum passes the reference by more than that (in
  // practice the first chunk, and rarely later) does the wave move it and rescale the
  // accumulators. The result, acc / lsum, does not depend on the reference.
  // A lane tests only its own eight logits of the row against the row's threshold thr[j] (a
  // raw logit whose weight would be 2^kSlack); the row maximum, which needs the four lanes of
  // the row, is formed only when some lane of the wave passes it.
  constexpr float kSlack = 8.0f;
  float m[2] = {-INFINITY, -INFINITY}, thr[2] = {-INFINITY, -INFINITY};
  f32x4 acc[2][NT], lsum[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lsum[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[j][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const V8 ones = __builtin_bit_cast(V8, u32x4{M::kOnePair, M::kOnePair, M::kOnePair, M::kOnePair});

  const int wave_first_limit = base + wt0;  // smallest limit among this wave's rows
  const int wave_last_limit = base + wt1;   // largest

  // masked: the chunk reaches past some row's limit of this wave (the causal edge, or
  // positions >= L).
  auto compute = [&](int n, int st, bool masked) {
    u32x4 kr[2][KK];
    u32x4 vr[NT];
    read_stage(st, kr, vr);
    const int pos0 = n * CT + 8 * r;  // this lane's first position of the chunk
    // Logits of both column tiles first, then one test for both: the part after it is one
    // straight run (exp, P, the PV products) that the compiler can interleave across the tiles.
    float sv[2][8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s0 = M::mac(__builtin_bit_cast(V8, kr[0][kk]), qb[j][kk], s0);
        s1 = M::mac(__builtin_bit_cast(V8, kr[1][kk]), qb[j][kk], s1);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[j][e] = s0[e];
        sv[j][4 + e] = s1[e];
      }
    }
    if (masked) {  // uniform: a branch, not a select on every chunk
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int lim = plim[j] - pos0;
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[j][e] = e <= lim ? sv[j][e] : -INFINITY;
      }
    }
    float x[2];  // -inf where the lane's positions lie past the row's limit
#pragma unroll
    for (int j = 0; j < 2; ++j)
      x[j] = fmaxf(fmaxf(fmaxf(sv[j][0], sv[j][1]), fmaxf(sv[j][2], sv[j][3])),
                   fmaxf(fmaxf(sv[j][4], sv[j][5]), fmaxf(sv[j][6], sv[j][7])));
    if (__builtin_amdgcn_ballot_w64(x[0] > thr[0] || x[1] > thr[1])) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float y = across16(x[j], OpMax());
        y = across32(y, OpMax());
        const float mnew = fmaxf(m[j], y * cl);  // finite: every row sees position 0 first
        const float alpha = __builtin_amdgcn_exp2f(m[j] - mnew);
        m[j] = mnew;
        thr[j] = (mnew + kSlack) / cl;  // +inf when cl = 0: every weight is then 2^-m
        lsum[j] *= alpha;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[j][nt] *= alpha;
      }
    }
    wait_v(vr);
    // Positions at or past L may hold anything (even NaN): zero their V, 0 * NaN is NaN.
    const int nv = L - pos0;
    if (masked && n * CT + CT > L && nv < 8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t keep = (2 * q + 1 < nv) ? 0xffffffffu : (2 * q < nv) ? 0x0000ffffu : 0u;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) vr[nt][q] &= keep;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      V8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[e] = M::narrow(__builtin_amdgcn_exp2f(fmaf(sv[j][e], cl, -m[j])));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[j][nt] = M::mac(__builtin_bit_cast(V8, vr[nt]), pb, acc[j][nt]);
      lsum[j] = M::mac(ones, pb, lsum[j]);
    }
  };

  // A ring of four stages, chunk n in stage n % 4, loaded three chunks ahead. Before the
  // barrier of step n this wave waits for its own loads of chunk n; after it, every wave's
  // loads of chunk n are in and every wave is done with chunk n - 1, whose stage then takes
  // chunk n + 3.
  static_assert(kStages == 4, "one chunk per step, three chunks ahead");
  for (int k = 0; k < 3 && k < nch; ++k) issue(k, k);
#pragma unroll 1
  for (int n = 0; n < nch; ++n) {
    // This wave's loads of chunk n are done when at most those of the chunks after it that
    // were issued (up to two) are still in flight.
    if (n + 2 < nch) wait_vm_le<2 * LPW>();
    else if (n + 1 < nch) wait_vm_le<LPW>();
    else wait_vm_le<0>();
    stage_barrier();
    if (n + 3 < nch) issue(n + 3, (n + 3) % kStages);
    if (wave_live && n * CT <= wave_last_limit)
      compute(n, n % kStages, n * CT + CT - 1 > wave_first_limit);
  }

  // Lane (r, c) holds O^T[16 nt + 4 r + e][row c] of each column tile, and the row's whole
  // softmax sum.
  if (!wave_live) return;
  T* out = reinterpret_cast<T*>(a.out);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (!valid[j]) continue;
    const float inv = 1.0f / lsum[j][0];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      T v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = from_f32<DT>(acc[j][nt][e] * inv);
      *reinterpret_cast<u32x2*>(out + orow[j] + 16 * nt + 4 * r) = __builtin_bit_cast(u32x2, v4);
    }
  }
}

template <Dt DT, int D, int S>
hipError_t launch_s(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_units * p.num_kv_heads);
  prefill_kernel<DT, D, S><<<grid, dim3(kPrefillWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

template <Dt DT, int D>
hipError_t launch_d(int block_size, const PrefillParams& p, hipStream_t stream) {
  switch (block_size) {
    case 16: return launch_s<DT, D, 16>(p, stream);
    case 32: return launch_s<DT, D, 32>(p, stream);
    case 64: return launch_s<DT, D, 64>(p, stream);
    case 128: return launch_s<DT, D, 128>(p, stream);
    case 256: return launch_s<DT, D, 256>(p, stream);
    default: return hipErrorNotSupported;
  }
}

template <Dt DT>
hipError_t launch_t(int head_dim, int block_size, const PrefillParams& p, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<DT, 64>(block_size, p, stream);
    case 128: return launch_d<DT, 128>(block_size, p, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_prefill(Dt dt, int head_dim, int block_size, const PrefillParams& p,
                          hipStream_t stream) {
  switch (dt) {
    case Dt::F16: return launch_t<Dt::F16>(head_dim, block_size, p, stream);
    case Dt::BF16: return launch_t<Dt::BF16>(head_dim, block_size, p, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pkv
