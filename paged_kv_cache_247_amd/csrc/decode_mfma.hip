// Paged decode attention with gfx950 matrix cores, for fp16/bf16 when a grouped-query group of
// G >= 4 query heads shares each kv head: per 32-position chunk the logits are a dense
// [32 x D] by [D x G] product and the output update a dense [D x 32] by [32 x G] product.
// The G heads are the 16 columns of v_mfma_f32_16x16x32_{bf16,f16} (G <= 16; unused columns
// hold zero queries and are never written).
//
// The operation is attention over non-contiguous KV-cache blocks (vAttention, section 3.1
// "Requires re-writing the attention kernel"; grouped-query attention is the case that
// section singles out), each block reached through the block table (Qualiteg, "About
// PagedAttention for LLM serving", "There are logical blocks and physical blocks ...") and each
// sequence using only its own length (same post, item 2-1).
//
// Register layouts (lane = 16 r + c, r in 0..3, c in 0..15). For a 16x16x32 product the A
// operand gives lane (r, c) row c and eight consecutive k values of group r, the B operand
// column c and the same eight k values, and the accumulator holds rows 4r..4r+3 of column c.
// Only the pairing of A's and B's k values matters, so k is mapped freely:
//   logits   S^T[t][h] = sum_d K[t][d] q[h][d]      A = K rows, B = q columns
//     lane (r, c) loads K row tau = 8(c/4) + 4 gi + (c%4) (gi = 0, 1 picks one of two
//     products) at d = 32 kk + 8r .. +8, so its accumulator holds positions 8r .. 8r+7 of
//     head c, in order.
//   output   O^T[d][h] = sum_t V^T[d][t] P^T[t][h]  A = V^T rows, B = softmax weights
//     lane (r, c) loads V^T row d = 16 nt + c at positions 8r .. 8r+7 -- 16 contiguous bytes
//     of the chunk's [D][32] column group (two [D][16] tiles at block size 16) -- and its B
//     operand is exactly the eight weights it computed.
//   The accumulator of tile nt holds O^T[16 nt + 4r + i][c]: the head is the lane's own
//   column, so the online-softmax rescale uses the lane's own running max; no exchange.
#include <type_traits>

#include "kernels.hpp"

#ifndef PKV_BLOCK_SIZE
#error "build once per block size with -DPKV_BLOCK_SIZE=16|32|64|128|256"
#endif

namespace pkv {
namespace {

template <Dt DT> struct Mfma;
template <> struct Mfma<Dt::BF16> {
  using V8 = bf16x8;
  static __device__ __forceinline__ f32x4 mac(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ __bf16 narrow(float x) { return (__bf16)x; }
};
template <> struct Mfma<Dt::F16> {
  using V8 = f16x8;
  static __device__ __forceinline__ f32x4 mac(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ _Float16 narrow(float x) { return (_Float16)x; }
};

// Waits until at most N vector memory operations of this wave are outstanding. The waitcnt
// intrinsic touches no memory, so it does not count as a store that could alias the block
// table (which keeps the table reads scalar); the scheduling barriers keep the LDS reads that
// depend on the wait below it.
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt fields (gfx9): vmcnt[3:0] and [15:14], expcnt[6:4] (7 = no wait), lgkmcnt[11:8]
  // (15 = no wait).
  constexpr int kEnc = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kEnc);
  __builtin_amdgcn_sched_barrier(0);
}

// Dword 3 of a raw buffer descriptor on gfx9-family chips: 32-bit data format, no swizzle,
// no index stride.
constexpr int kXcds = 8;  // XCDs of the MI355X, which take workgroups round robin
constexpr int kBufferFlags = 0x00020000;

// LDS of a decode workgroup: two K staging slots per wave (after the chunk loop the merge
// buffers), the newest position's logits and its V row.
template <int D, int NW>
struct DecodeLds {
  __attribute__((aligned(16))) char stage[NW * 2 * 32 * D * 2];
  float new_logit[16];
  float new_v[4 * D];  // the newest V row of each member of a group (of the sequence: row 0)
};

// x_k of four values, for a k that may differ between lanes: the values are taken by value so
// that they stay in registers (selecting among the fields of one object can be turned into an
// indexed load, which puts the object in scratch memory).
__device__ __forceinline__ int pick4(int k, int x0, int x1, int x2, int x3) {
  int r = x3;
  r = k == 2 ? x2 : r;
  r = k == 1 ? x1 : r;
  r = k == 0 ? x0 : r;
  return r;
}

// One workgroup's unit: w is its index in the launch's numbering (below).
// GRP: a unit is a group of sequences whose block tables agree over the first range (a shared
// prefix); column c of the products is head c % G of member c / G, so each shared tile is read
// once for every member, and the range's partial state is written for each member.
// WG (GRP without PARTIAL): a unit is a whole group -- its members agree over the first
// range_tokens positions, which are read once for all members (every column), and then each
// member's own positions past them through its own table row (that member's columns only); the
// unit writes each member's output.
template <Dt DT, int D, int S, int NW, bool PARTIAL, bool NTL, bool TBL, bool GRP>
__device__ __forceinline__ void decode_unit(const DecodeParams& a, const int w,
                                            DecodeLds<D, NW>& lds) {
  static_assert(!GRP || TBL, "groups read through block tables");
  constexpr bool WG = GRP && !PARTIAL;
  static_assert(!WG || !NTL, "whole groups keep the shared tiles in L2 (cached loads)");
  static_assert(DT == Dt::BF16 || DT == Dt::F16, "16-bit inputs only");
  constexpr int EB = 2;
  constexpr int CT = 32;        // positions per chunk
  constexpr int BPC = S < CT ? CT / S : 1;  // blocks per chunk
  constexpr int CPK = S > CT ? S / CT : 1;  // chunks per block
  constexpr int KK = D / 32;    // k-steps of the logits product
  constexpr int NT = D / 16;    // 16-row tiles of the output product
  static_assert(BPC * S == CT || CPK * CT == S, "block_size 16, 32, 64, 128 or 256");
  using M = Mfma<DT>;
  using V8 = typename M::V8;
  using T = typename Elt<DT>::T;

  // K of a chunk is staged in LDS: each wave owns two slots of CT rows; a row's sixteen-byte
  // pieces are rotated by rot(t) so that the operand reads below hit distinct banks. After the
  // chunk loop the same space holds the merge buffers.
  constexpr int RB = D * EB;        // bytes of one K row
  constexpr int NPC = RB / 16;      // sixteen-byte pieces per K row
  constexpr int SLOT = CT * RB;     // one chunk of K
  constexpr int KLD = SLOT / 1024;  // 1 KiB direct-to-LDS loads per chunk
  // Accumulator rows are padded by 16 bytes: lanes of one row group write the same columns of
  // sixteen different head rows, which must not share banks.
  constexpr int DP = D + 4;
  static_assert((NW * 16 * DP + 2 * NW * 16) * 4 <= NW * 2 * SLOT, "merge fits the staging area");
  static_assert(sizeof(lds.stage) == NW * 2 * SLOT, "staging slots");
  char* const smem = lds.stage;
  float* const sh_new = lds.new_logit;
  float* const sh_vnew = lds.new_v;
  auto sh_acc = reinterpret_cast<float (*)[16][DP]>(smem);
  auto sh_m = reinterpret_cast<float (*)[16]>(smem + NW * 16 * DP * 4);
  auto sh_l = reinterpret_cast<float (*)[16]>(smem + (NW * 16 * DP + NW * 16) * 4);

  const int Hkv = a.num_kv_heads;
  const int H = a.num_heads;
  const int G = H / Hkv;
  const int MB = a.max_blocks_per_seq;
  // Workgroups go to the XCDs round robin (w % 8). Unshared KV: every kv head of a unit on one
  // XCD (groups of 8 Hkv workgroups hold 8 units, head g of the group's unit j at 8 g + j), so
  // an XCD streams whole blocks of its sequences. Shared prefix blocks (cached loads): head g of
  // every unit on XCD g % 8, so a shared block's head tile stays in one XCD's L2.
  int g, slot;
  if constexpr (NTL) {
    constexpr int XC = kXcds;
    g = (w % (XC * Hkv)) / XC;
    slot = (w / (XC * Hkv)) * XC + w % XC;
    if (slot >= a.num_units) return;  // the grid is padded to whole groups of 8 units
  } else {
    g = w % Hkv;
    slot = w / Hkv;
    if (slot >= a.num_units) return;  // a combined grid pads each kind to whole groups of 8
  }
  int unit = a.work_items ? a.work_items[slot] : slot;
  unit = min(max(unit, 0), (GRP ? a.num_units : a.num_seqs * a.num_ranges) - 1);
  const int part = GRP ? 0 : unit % a.num_ranges;
  // GRP: the group's row of four members in one 16-byte load (rows are 16-byte aligned), so
  // that the loads which depend on it all issue together instead of one after another. The
  // first member's table row and length stand for the group's (they agree over the range by the
  // caller's contract).
  u32x4 grow = {0u, 0u, 0u, 0u};
  if constexpr (GRP) grow = *reinterpret_cast<const u32x4*>(a.group_members + 4 * unit);
  const int i = GRP ? min(max((int)grow[0], 0), a.num_seqs - 1) : unit / a.num_ranges;
  auto wm_of = [&](int k) {  // GRP: member k of the group, -1 for none
    const int m = pick4(k, (int)grow[0], (int)grow[1], (int)grow[2], (int)grow[3]);
    return k * G < 16 && m >= 0 && m < a.num_seqs ? m : -1;
  };
  // Columns in use: the G heads, or G heads of each of up to 16 / G group members.
  const int ncol = GRP ? 16 : G;
  const int lane = lane_id();
  const int wave = wave_id();
  const int r = lane >> 4;
  const int c = lane & 15;
  // q columns: lane (r, c) holds head c at d = 32 kk + 8r .. +8; in GRP mode head c % G of
  // member c / G. Columns past the group's heads (or of a missing member) load some valid q row
  // instead of zeros: the columns are independent and their results are never written, and
  // unconditional loads let the compiler count them in its waits instead of waiting for all.
  // These loads and the new rows below depend only on the unit, so they go out before the
  // lengths and block ids the first chunk waits for.
  auto column_seq = [&](int col) {
    if constexpr (GRP) {
      const int s = col / G;
      const int m = s < 4 ? (int)pick4(s, grow[0], grow[1], grow[2], grow[3]) : -1;
      return m < a.num_seqs ? m : -1;
    } else {
      return col < G ? i : -1;
    }
  };
  V8 qb[KK];
  {
    const int qs = column_seq(c);
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((size_t)(GRP ? max(qs, 0) : i) * H + (size_t)g * G + c % G) * D + 8 * r) *
                         EB;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qb[kk] = __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(qp + kk * 64));
  }

  // Position L-1 joins the merge below as one more partial state (m = its logit, l = 1,
  // acc = its V row). Its rows are loaded before the first chunk (vector loads return in
  // order, so waiting for them below does not wait for the chunk).
  // WG: every member's newest position; the K row pieces of member k go to lanes
  // k * PPR .. k * PPR + PPR - 1, and lane (r, c)'s logit pieces are those of its column's
  // member.
  constexpr int NMEM = WG ? 4 : 1;   // newest rows per unit
  constexpr int PPR = D * EB / 16;   // sixteen-byte pieces per K row
  auto new_row = [&](int seq) {      // this kv head's newest K row of sequence seq, in bytes
    return reinterpret_cast<const char*>(a.new_key) + ((size_t)seq * Hkv + g) * D * EB;
  };
  const char* kn = new_row(i);
  const T* vn = reinterpret_cast<const T*>(a.new_value) + ((size_t)i * Hkv + g) * D;
  // Set only in the waves that use them (no default value: a merge of a loaded value with a
  // default makes the compiler copy, and so wait for, the load right where it is issued).
  u32x4 kpiece[KK];
  u32x4 krow;
  T vrow[D / 64];  // the sequence's V row (not WG)
  u32x4 vrow4;     // WG: sixteen-byte piece lane % PPR of member lane / PPR's V row
  // Block of the newest position: one per lane (lane k: member k's), so that the load stays a
  // vector load that nothing waits for until the stores at the end (a uniform one would be
  // moved to a scalar register, with a wait, as soon as it is issued).
  int slot_blk;
  // The rows depend on the unit only (in split mode on the range too: there they are loaded
  // once the length is known). Every load is unconditional: lanes past a row's pieces and
  // missing members read rows that exist (the stores skip them; publish_new_rows zeroes a
  // missing member's V).
  auto load_new_rows = [&]() {
    if (wave == NW - 1) {
      const char* kp = WG ? new_row(max(column_seq(c), 0)) : kn;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kpiece[kk] = *reinterpret_cast<const u32x4*>(kp + (32 * kk + 8 * r) * EB);
    }
    if (wave == 0) {
      // WG: the members' V rows in one load, laid out like their K rows below.
      const int km = min(lane / PPR, NMEM - 1);
      if constexpr (WG) {
        const int m = max(wm_of(km), 0);
        vrow4 = reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(a.new_value) + ((size_t)m * Hkv + g) * D * EB)[lane % PPR];
      } else {
#pragma unroll
        for (int e = 0; e < D / 64; ++e) vrow[e] = vn[lane + 64 * e];
      }
      krow = reinterpret_cast<const u32x4*>(WG ? new_row(max(wm_of(km), 0)) : kn)[lane % PPR];
    }
  };
  if ((WG || !PARTIAL) && a.new_key != nullptr) load_new_rows();

  // Physical block of logical block j: the sequence's table entry (TBL), or without tables the
  // contiguous reservation of MB blocks per sequence (block i * MB + j).
  const int32_t* bt = a.block_tables + (size_t)i * MB;
  const int contig0 = i * MB;
  const int start = part * a.range_tokens;

  // Waves take chunks wave, wave + NW, ... of the range: local chunk m of this wave is chunk
  // n = wave + NW m, which covers logical blocks start / S + n BPC + e, e < BPC (blocks of 16
  // or 32 positions), or rows (n % CPK) CT .. + CT of logical block start / S + n / CPK (larger
  // blocks). The wave keeps the ids of CPB consecutive local chunks in one register, lane
  // BPC (m % CPB) + e holding block e of local chunk m, and picks them out with readlane. One
  // coalesced vector load fills it every CPB chunks. (The block table cannot be read through
  // the scalar cache inside the loop: the direct-to-LDS loads count as writes to unknown
  // memory, which rules scalar loads out.)
  // The first batch is loaded now, in parallel with the context length; any entry of the row
  // may be read and ids are clamped into the pool before use.
  constexpr int CPB = 64 / BPC;

  // WG: members (up to 16 / G, -1 for none), their lengths and ends of their own positions
  // (L - 1 with a fused write), and how many chunks each has past the shared P positions.
  // Chunk v of the unit's list is, while both kinds last, shared chunk v / 2 for even v and
  // member chunk v / 2 for odd v -- shared chunks come from L2, members' chunks from HBM, and
  // mixing them keeps both busy -- then the rest of whichever kind is left; member chunks are
  // member 0's, then member 1's, and so on.
  // (Four named values per quantity rather than arrays: indexed by a lane's member, an array
  // would live in scratch memory.)
  struct Four {
    int v0, v1, v2, v3;
    __device__ __forceinline__ int operator[](int k) const { return pick4(k, v0, v1, v2, v3); }
  };
  Four wm = {-1, -1, -1, -1}, wL = {0, 0, 0, 0}, wE = {0, 0, 0, 0}, wcum = {0, 0, 0, 0};
  int wP = 0, wNS = 0, wNM = 0;
  if constexpr (WG) {
    wm = {wm_of(0), wm_of(1), wm_of(2), wm_of(3)};
    // The four lengths load unconditionally (a missing member reads sequence 0's) and are
    // masked after, so they too are one round trip (the empty asm keeps the compiler from
    // moving each load back under its member's condition, one wait after another).
    int x0 = a.context_lens[max(wm.v0, 0)], x1 = a.context_lens[max(wm.v1, 0)];
    int x2 = a.context_lens[max(wm.v2, 0)], x3 = a.context_lens[max(wm.v3, 0)];
    asm volatile("" : "+s"(x0), "+s"(x1), "+s"(x2), "+s"(x3));
    auto len = [&](int m, int x) { return m >= 0 ? min(max(x, 0), MB * S) : 0; };
    wL = {len(wm.v0, x0), len(wm.v1, x1), len(wm.v2, x2), len(wm.v3, x3)};
    wP = min(max(a.range_tokens, 0), MB * S);
    wNS = wm.v0 >= 0 ? (wP + CT - 1) / CT : 0;
    const int nf = a.new_key != nullptr ? 1 : 0;
    wE = {max(wL.v0 - nf, 0), max(wL.v1 - nf, 0), max(wL.v2 - nf, 0), max(wL.v3 - nf, 0)};
    auto own = [&](int e) { return e > wP ? (e - wP + CT - 1) / CT : 0; };
    wcum.v0 = own(wE.v0);
    wcum.v1 = wcum.v0 + own(wE.v1);
    wcum.v2 = wcum.v1 + own(wE.v2);
    wcum.v3 = wcum.v2 + own(wE.v3);
    wNM = wcum.v3;
  }
  struct ChunkInfo {
    int row;  // sequence whose table row holds the chunk's blocks
    int cs;   // the chunk's first position
    int ce;   // end of the positions of its range
    int k;    // member whose columns it feeds, -1 for all (shared)
  };
  auto chunk_info = [&](int v) {
    const int mn = min(wNS, wNM);
    int sh = -1, mi = -1;
    if (v < 2 * mn) {
      if (v & 1) mi = v >> 1;
      else sh = v >> 1;
    } else if (wNS > wNM) {
      sh = v - mn;
    } else {
      mi = v - mn;
    }
    ChunkInfo ci;
    if (sh >= 0) {
      ci.row = wm.v0;
      ci.cs = sh * CT;
      ci.ce = wP;
      ci.k = -1;
    } else {
      const int k = (mi >= wcum.v0) + (mi >= wcum.v1) + (mi >= wcum.v2);
      const int base = k == 0 ? 0 : wcum[k - 1];
      ci.row = wm[k];
      ci.cs = wP + (mi - base) * CT;
      ci.ce = wE[k];
      ci.k = k;
    }
    ci.row = max(ci.row, 0);
    return ci;
  };

  auto load_id_batch = [&](int kb) {
    const int n = wave + NW * (kb * CPB + lane / BPC);
    if constexpr (WG) {
      if (n >= wNS + wNM) return 0;
      const ChunkInfo ci = chunk_info(n);
      const int blk = ci.cs / S + (BPC == 2 ? lane % BPC : 0);
      return blk < MB ? a.block_tables[(size_t)ci.row * MB + blk] : 0;
    } else {
      const int blk = start / S + (BPC == 2 ? n * BPC + lane % BPC : n / CPK);
      return blk < MB ? bt[blk] : 0;
    }
  };
  if (WG && a.new_key != nullptr && wave == 0) {
    const int ks = min(lane, NMEM - 1);
    slot_blk = a.block_tables[(size_t)max(wm[ks], 0) * MB + (max(wL[ks], 1) - 1) / S];
  }
  int id_batch = 0;
  if constexpr (TBL) id_batch = load_id_batch(0);

  int L = WG ? wL.v0 : a.context_lens[i];
  L = min(max(L, 0), MB * S);
  if (!WG && start >= L) {
    if (!PARTIAL && part == 0) {
      T* o = reinterpret_cast<T*>(a.out) + ((size_t)i * H + (size_t)g * G) * D;
      for (int e = threadIdx.x; e < G * D; e += NW * 64) o[e] = from_f32<DT>(0.0f);
    }
    return;
  }
  // With a fused write, position L-1 comes from new_key/new_value (this is then the sequence's
  // last range) and the cache is read only up to L-2. (WG: each member's position L - 1.)
  const bool fused = a.new_key != nullptr && (WG || start + a.range_tokens >= L);
  const int end = min(start + a.range_tokens, L) - (fused ? 1 : 0);
  const int nch = WG ? wNS + wNM : max(end - start + CT - 1, 0) / CT;
  const int blk_end = (end + S - 1) / S;  // first logical block past the cached range

  const size_t tile_bytes = (size_t)S * D * EB;
  const size_t id_stride = (size_t)Hkv * tile_bytes;
  const char* kpool = reinterpret_cast<const char*>(a.k_cache) + (size_t)g * tile_bytes;
  const char* vpool = reinterpret_cast<const char*>(a.v_cache) + (size_t)g * tile_bytes;
  // K: this lane's operand rows are chunk positions t = 8(c/4) + (c%4) (+4 for the second
  // product), pieces 4 kk + r.
  const int k_tau = 8 * (c >> 2) + (c & 3);
  // V^T: row d = 16 nt + c, positions 8r .. 8r+7 of the chunk (in block 8r / S when a chunk
  // spans two blocks). A block stores V in column groups of VS positions, each a [D][VS]
  // tile; a chunk of a larger block is exactly one group, ro D elements into the block.
  constexpr int VS = S < CT ? S : CT;
  const int v_blk = (8 * r) / S;
  const int v_off = c * VS * EB + ((8 * r) % S) * EB;  // + nt * 16 rows

  struct Ids {
    int b0, b1;
    int ro;  // first row of the chunk within block b0 (nonzero only for blocks over 32)
    int cs, ce, k;  // WG: the chunk's first position, its range's end, its member (-1: shared)
    // This lane's V^T pieces of the chunk, formed with the ids a step early; pieces 4 KiB and
    // more past vt are addressed from vt4 (= vt + 4 KiB, the reach of an immediate offset).
    const char* vt;
    const char* vt4;
  };
  auto clamp_id = [&](int id) { return min(max(id, 0), a.num_blocks - 1); };
  // Physical ids of local chunk m's blocks; a second block past the range reuses the first (its
  // positions are masked). Called for m = 0, 1, 2, ... in order.
  auto fetch_ids = [&](int m) {
    const int n = wave + NW * m;
    Ids ids;
    int b0, bend;  // the chunk's first logical block; the first block past its range
    if constexpr (WG) {
      const ChunkInfo ci = chunk_info(n);
      b0 = ci.cs / S;
      ids.ro = CPK > 1 ? ci.cs % S : 0;
      bend = (ci.ce + S - 1) / S;
      ids.cs = ci.cs;
      ids.ce = ci.ce;
      ids.k = ci.k;
    } else {
      b0 = start / S + (BPC == 2 ? n * BPC : n / CPK);
      ids.ro = (n % CPK) * CT;
      bend = blk_end;
      ids.cs = ids.ce = ids.k = 0;
    }
    if constexpr (TBL) {
      if (m > 0 && m % CPB == 0) {
        id_batch = load_id_batch(m / CPB);
        // Wait for the refill inside this rarely taken branch: a use here makes the compiler
        // place its vmcnt wait now instead of before every readlane after the branches merge.
        asm volatile("" : "+v"(id_batch));
      }
      const int sel = (m % CPB) * BPC;
      ids.b0 = clamp_id(__builtin_amdgcn_readlane(id_batch, sel));
      ids.b1 = (BPC == 2 && b0 + 1 < bend)
                   ? clamp_id(__builtin_amdgcn_readlane(id_batch, sel + 1))
                   : ids.b0;
    } else {
      ids.b0 = clamp_id(contig0 + b0);
      ids.b1 = (BPC == 2 && b0 + 1 < bend) ? clamp_id(contig0 + b0 + 1) : ids.b0;
    }
    ids.vt = vpool + (size_t)(v_blk ? ids.b1 : ids.b0) * id_stride + (size_t)ids.ro * D * EB +
             v_off;
    ids.vt4 = ids.vt + 4096;
    return ids;
  };

  struct Regs {
    u32x4 v[NT];
    int cs, ce, k;  // WG: the chunk these registers hold (see Ids)
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

  // Chunk loads: K with KLD coalesced 1 KiB buffer loads straight into the wave's LDS slot
  // (lane l of load x fills row t = x * (1024 / RB) + l / NPC, rotated piece l % NPC), V^T
  // straight into registers (16 contiguous bytes per lane). Each K block tile gets its own
  // buffer descriptor (uniform, built with scalar arithmetic), so 32-bit offsets reach any
  // pool size. The buffer form (rather than the global one) matters: the compiler counts it
  // as an in-order vector memory operation, while a global load into LDS makes it flush the
  // whole counter at every later wait.
  static_assert(S % (1024 / RB) == 0, "a 1 KiB load stays within one block");
  auto tile_rsrc = [&](int id, int ro) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kpool + (size_t)id * id_stride + (size_t)ro * RB), 0,
        (int)tile_bytes - ro * RB, kBufferFlags);
  };
  auto load_as = [&](const Ids& ids, Regs& R, int slot, auto nt, auto knt) {
    constexpr bool NTC = decltype(nt)::value;   // every load non-temporal
    constexpr bool KNT = decltype(knt)::value;  // the K loads non-temporal
    char* dst = smem + (wave * 2 + slot) * SLOT;
    const __amdgpu_buffer_rsrc_t r0 = tile_rsrc(ids.b0, ids.ro);
    const __amdgpu_buffer_rsrc_t r1 = BPC == 2 ? tile_rsrc(ids.b1, 0) : r0;
#pragma unroll
    for (int x = 0; x < KLD; ++x) {
      const int t = x * (1024 / RB) + lane / NPC;
      const int jt = (lane % NPC - rot(t)) & (NPC - 1);
      const bool second = BPC == 2 && x * (1024 / RB) >= S;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          second ? r1 : r0, (__attribute__((address_space(3))) void*)(dst + x * 1024), 16,
          (t % S) * RB + jt * 16, 0, 0, (NTC || KNT) ? 2 : 0);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      constexpr int kStep = 16 * VS * EB;
      const int off = nt * kStep;
      R.v[nt] = load_kv<NTC, u32x4>(off < 4096 ? ids.vt + off : ids.vt4 + (off - 4096));
    }
  };
  auto load = [&](const Ids& ids, Regs& R, int slot, auto knt) {
    if constexpr (WG) {
      R.cs = ids.cs;
      R.ce = ids.ce;
      R.k = ids.k;
    }
    load_as(ids, R, slot, std::integral_constant<bool, NTL>(), knt);
  };
  // Operand pieces of chunk K from the wave's slot. The reads are issued as inline LDS
  // instructions that the compiler does not see as LDS reads, so it adds no waits of its own
  // for the loads in flight into the other slot; the caller's vmcnt wait has made this slot's
  // data visible, and the lgkmcnt wait below completes the reads before their results are used.
  auto read_k = [&](int slot, u32x4 (&kr)[2][KK]) {
    const char* src = smem + (wave * 2 + slot) * SLOT;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int t = k_tau + 4 * gi;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(
            src + t * RB + ((4 * kk + r + rot(t)) & (NPC - 1)) * 16);
        asm volatile("ds_read_b128 %0, %1" : "=v"(kr[gi][kk]) : "v"(addr) : "memory");
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(kr[gi][kk]));
  };

  float m = -INFINITY, l = 0.0f;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Chunk n from the registers R and LDS slot. Only a wave's last chunk can reach past the end
  // of the range (chunks are dealt round robin), so only that one (last = true) masks.
  auto compute = [&](int n, Regs& R, int slot, auto last) {
    // WG: chunks of any range can be partial, so every chunk masks; a member's chunk feeds
    // only that member's columns (the others see no position in it).
    constexpr bool MASK = WG || decltype(last)::value;
    const int cbase = WG ? R.cs : start + n * CT;
    const int cend = WG ? R.ce : end;
    const bool active = !WG || R.k < 0 || c / G == R.k;
    u32x4 kr[2][KK];
    read_k(slot, kr);
    f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = M::mac(__builtin_bit_cast(V8, kr[0][kk]), qb[kk], s0);
      s1 = M::mac(__builtin_bit_cast(V8, kr[1][kk]), qb[kk], s1);
    }
    const int pos0 = cbase + 8 * r;  // position of this lane's first logit
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sv[j] = (!MASK || (pos0 + j < cend && active)) ? sv[j] * a.scale_log2e : -INFINITY;
      mx = fmaxf(mx, sv[j]);
    }
    mx = across16(mx, OpMax());
    mx = across32(mx, OpMax());
    const float mnew = fmaxf(m, mx);
    // WG: a column that has seen no position yet keeps m = -inf; offsetting by 0 instead keeps
    // its weights and rescale at 0 rather than NaN.
    const float mref = WG && mnew == -INFINITY ? 0.0f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - mref);
    m = mnew;
    V8 pb;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pb[j] = M::narrow(__builtin_amdgcn_exp2f(sv[j] - mref));
      psum += (float)pb[j];  // the sum matches the weights the product uses
    }
    l = fmaf(l, alpha, psum);
    // Positions past the end may hold anything (even NaN): zero them, 0 * NaN is NaN.
    const int nv = cend - pos0;
    if (MASK && nv < 8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t keep = (2 * q + 1 < nv) ? 0xffffffffu : (2 * q < nv) ? 0x0000ffffu : 0u;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) R.v[nt][q] &= keep;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[nt] *= alpha;
      acc[nt] = M::mac(__builtin_bit_cast(V8, R.v[nt]), pb, acc[nt]);
    }
  };

  // Position L-1 joins the merge below as one more partial state (m = its logit, l = 1,
  // acc = its V row). Its rows are loaded before the first chunk (vector loads return in
  // order, so waiting for them below does not wait for the chunk).
  // WG: every member's newest position; the K row pieces of member k go to lanes
  // k * PPR .. k * PPR + PPR - 1, and lane (r, c)'s logit pieces are those of its column's
  // member.
  if (!WG && fused) {
    if (PARTIAL) load_new_rows();
    // Lane 0's entry is the one used; the others read neighbours in the row, which keeps this
    // a vector load.
    if (wave == 0)
      slot_blk = TBL ? bt[min((L - 1) / S + lane, MB - 1)] : contig0 + (L - 1) / S;
  }

  // The new position's logits (the last wave: a register per lane, computed once the first
  // chunk's loads are out) and, after the chunk loop, the LDS copies the merge reads: the
  // logits and the V rows. LDS writes while direct-to-LDS loads are in flight would make the
  // compiler wait for those loads (they count as LDS writes), so none are made before the loop.
  float nlogit = 0.0f;
  auto new_logit = [&]() {
    if (wave == NW - 1) {
      // The empty asm statements keep this after the first chunk's loads (the compiler would
      // otherwise let it precede them, waiting there for the new rows).
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(kpiece[kk]) : : "memory");
      // Logit of head c: fp32 dot over the d pieces this lane holds of q, summed over rows.
      float part_dot = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const V8 kv = __builtin_bit_cast(V8, kpiece[kk]);
#pragma unroll
        for (int j = 0; j < 8; ++j) part_dot = fmaf((float)qb[kk][j], (float)kv[j], part_dot);
      }
      part_dot = across16(part_dot, OpAdd());
      nlogit = across32(part_dot, OpAdd()) * a.scale_log2e;
    }
  };
  auto publish_new_rows = [&]() {
    if (wave == NW - 1 && r == 0 && c < ncol) sh_new[c] = nlogit;
    if (wave == 0) {
      if constexpr (WG) {
        const int k = lane / PPR;  // lanes past the four members' pieces hold copies
        const bool has = wm[min(k, NMEM - 1)] >= 0 && wL[min(k, NMEM - 1)] > 0;
        const V8 x = __builtin_bit_cast(V8, vrow4);
        if (k < NMEM) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sh_vnew[k * D + (lane % PPR) * 8 + j] = has ? (float)x[j] : 0.0f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < D / 64; ++e) {
          const int d = lane + 64 * e;
          if constexpr (DT == Dt::BF16) sh_vnew[d] = bits_f((uint32_t)vrow[e] << 16);
          else sh_vnew[d] = (float)vrow[e];
        }
      }
    }
  };

  // WG: the members' own K streams from HBM with the non-temporal policy, so that it does not
  // push the shared tiles out of L2 (V loads stay ordinary). The policy is an immediate of the
  // load instruction, and a choice per chunk (a branch around the loads) makes the compiler
  // lose count of the loads in flight, so that it waits for the next chunk's K before
  // computing the current one. So the policy is the wave's, for its whole loop (two copies of
  // the loop): while both kinds of chunks last, the odd waves take the own chunks and the even
  // ones the shared chunks (the order of the list above), and of the chunks left after that,
  // of one kind, the odd waves load theirs non-temporal.
  int n = wave;
  auto chunk_loop = [&](auto knt) {
    Regs A, B;
    Ids ids = fetch_ids(0);
    int m_next = 1;  // local index of the chunk whose ids are fetched next
    load(ids, A, 0, knt);
    if (n + NW < nch) ids = fetch_ids(m_next++);
    if (fused) new_logit();
    // Two stages: chunk n + NW loads while chunk n computes; its block ids were fetched one
    // step earlier still. The LDS half of a chunk is not tracked by the compiler, so each
    // step waits explicitly: vector memory operations complete in order, and exactly
    // KLD + NT of them (the next chunk's) may still be in flight when chunk n is read. Each
    // steady-state compute is reached only through the next chunk's loads and that wait, so
    // the compiler's own waits for the V registers count the same KLD + NT operations; the
    // last chunk is computed after a full wait.
    const std::false_type mid;
    const std::true_type last;
    while (true) {
      if (n + NW >= nch) {
        wait_vm_le<0>();
        compute(n, A, 0, last);
        break;
      }
      load(ids, B, 1, knt);
      if (n + 2 * NW < nch) ids = fetch_ids(m_next++);
      wait_vm_le<KLD + NT>();
      compute(n, A, 0, mid);
      n += NW;
      if (n + NW >= nch) {
        wait_vm_le<0>();
        compute(n, B, 1, last);
        break;
      }
      load(ids, A, 0, knt);
      if (n + 2 * NW < nch) ids = fetch_ids(m_next++);
      wait_vm_le<KLD + NT>();
      compute(n, B, 1, mid);
      n += NW;
    }
  };
  if (n < nch) {
    if constexpr (WG) {
      if (wave & 1) chunk_loop(std::true_type());
      else chunk_loop(std::false_type());
    } else {
      chunk_loop(std::false_type());
    }
  } else if (fused) {
    new_logit();
  }
  if (fused) publish_new_rows();

  l = across16(l, OpAdd());
  l = across32(l, OpAdd());

  __syncthreads();  // every wave is done with its staging slots: the merge buffers reuse them
  if (c < ncol) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) sh_acc[wave][c][16 * nt + 4 * r + e] = acc[nt][e];
    if (r == 0) {
      sh_m[wave][c] = m;
      sh_l[wave][c] = l;
    }
  }
  __syncthreads();

  for (int e = threadIdx.x; e < ncol * D; e += NW * 64) {
    const int h = e / D;  // column
    const int d = e % D;
    const int seq = GRP ? column_seq(h) : i;
    if (GRP && seq < 0) continue;
    float Mx = fused ? sh_new[h] : -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) Mx = fmaxf(Mx, sh_m[v][h]);
    if (WG && Mx == -INFINITY) {  // a member with no position at all: a zero row
      reinterpret_cast<T*>(a.out)[((size_t)seq * H + (size_t)g * G + h % G) * D + d] =
          from_f32<DT>(0.0f);
      continue;
    }
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float f = __builtin_amdgcn_exp2f(sh_m[v][h] - Mx);
      num = fmaf(f, sh_acc[v][h][d], num);
      den = fmaf(f, sh_l[v][h], den);
    }
    if (fused) {
      const float f = __builtin_amdgcn_exp2f(sh_new[h] - Mx);
      num = fmaf(f, sh_vnew[(WG ? h / G : 0) * D + d], num);
      den += f;
    }
    const float o = num / den;
    const size_t row = (size_t)seq * H + (size_t)g * G + (GRP ? h % G : h);
    if constexpr (PARTIAL) {
      const size_t rec = row * a.num_ranges + part;
      a.tmp_out[rec * D + d] = o;
      if (d == 0) {
        a.max_logits[rec] = Mx * kLn2;
        a.exp_sums[rec] = den;
      }
    } else {
      reinterpret_cast<T*>(a.out)[row * D + d] = from_f32<DT>(o);
    }
  }

  // The new rows go to the slot the table maps position L-1 to. The stores come last: after
  // every block-table read, so the table can stay in the scalar cache (a store that might alias
  // it would force those reads through the vector memory path), and after the merge, whose LDS
  // reads wait for every vector memory operation in flight (the direct-to-LDS loads count as
  // LDS writes), stores included.
  // WG: each member's rows (V read back from LDS, where it is stored exactly).
  if (fused && wave == 0) {
#pragma unroll
    for (int k = 0; k < NMEM; ++k) {
      const int Lk = WG ? wL[k] : L;
      if (WG && (wm[k] < 0 || Lk <= 0)) continue;
      const int p = Lk - 1;
      const size_t tile =
          ((size_t)clamp_id(__builtin_amdgcn_readlane(slot_blk, k)) * Hkv + g) * S * D;
      T* kc = reinterpret_cast<T*>(a.k_cache) + tile + (size_t)(p % S) * D;
      T* vc = reinterpret_cast<T*>(a.v_cache) + tile + (size_t)((p % S) / VS) * VS * D + p % VS;
      if (WG ? lane / PPR == k : lane < PPR)
        reinterpret_cast<u32x4*>(kc)[WG ? lane % PPR : lane] = krow;
#pragma unroll
      for (int e = 0; e < D / 64; ++e)
        vc[(size_t)(lane + 64 * e) * VS] =
            WG ? from_f32<DT>(sh_vnew[k * D + lane + 64 * e]) : vrow[e];
    }
  }
}

template <Dt DT, int D, int S, int NW, bool PARTIAL, bool NTL, bool TBL, bool GRP = false>
__global__ void __launch_bounds__(NW * 64)
decode_mfma_kernel(const DecodeParams a) {
  __shared__ DecodeLds<D, NW> lds;
  decode_unit<DT, D, S, NW, PARTIAL, NTL, TBL, GRP>(a, blockIdx.x, lds);
}

// A decode step over shared prefix blocks in one grid: the groups (grp, GRP units) and the
// step's other units (rest, a work list of (sequence, partition) units), both writing
// partials with cached loads. The grid is cut into pieces of 8 units (8 Hkv workgroups, head
// g of the piece's unit j at j Hkv + g: a kv head keeps the XCDs it has in the separate
// launches); pieces of groups and of other units alternate while both last, so the groups,
// which read their tiles from L2, run beside units that stream from HBM.
template <Dt DT, int D, int S, int NW>
__global__ void __launch_bounds__(NW * 64)
decode_mfma_shared_kernel(const DecodeParams grp, const DecodeParams rest) {
  __shared__ DecodeLds<D, NW> lds;
  const int per = kXcds * grp.num_kv_heads;  // workgroups per piece
  const int ng = (grp.num_units + kXcds - 1) / kXcds;
  const int nr = (rest.num_units + kXcds - 1) / kXcds;
  const int both = min(ng, nr);
  const int b = blockIdx.x / per;
  const int u = blockIdx.x - b * per;
  const bool grouped = b < 2 * both ? (b & 1) == 0 : ng > nr;
  const int kb = b < 2 * both ? b >> 1 : b - both;  // piece index within its kind
  if (grouped)
    decode_unit<DT, D, S, NW, true, false, true, true>(grp, kb * per + u, lds);
  else
    decode_unit<DT, D, S, NW, true, false, true, false>(rest, kb * per + u, lds);
}

constexpr int kMfmaWaves = 4;

template <Dt DT, int D, int S, bool PARTIAL, bool NTL>
hipError_t launch_p(const DecodeParams& p, hipStream_t stream) {
  const unsigned units = NTL ? (p.num_units + kXcds - 1) / kXcds * kXcds : p.num_units;
  const dim3 grid(units * (unsigned)p.num_kv_heads);
  const dim3 block(kMfmaWaves * 64);
  if (p.block_tables)
    decode_mfma_kernel<DT, D, S, kMfmaWaves, PARTIAL, NTL, true><<<grid, block, 0, stream>>>(p);
  else
    decode_mfma_kernel<DT, D, S, kMfmaWaves, PARTIAL, NTL, false><<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

// Groups sharing a prefix: partials, cached loads (a shared tile is read by every group of
// the XCD its kv head maps to), one workgroup per (group, kv head).
template <Dt DT, int D, int S>
hipError_t launch_grouped(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_units * (unsigned)p.num_kv_heads);
  decode_mfma_kernel<DT, D, S, kMfmaWaves, true, false, true, true>
      <<<grid, dim3(kMfmaWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

template <Dt DT, int D, int S>
hipError_t launch_combined(const DecodeParams& grp, const DecodeParams& rest,
                           hipStream_t stream) {
  const unsigned pieces = (unsigned)(grp.num_units + kXcds - 1) / kXcds +
                          (unsigned)(rest.num_units + kXcds - 1) / kXcds;
  const dim3 grid(pieces * kXcds * (unsigned)grp.num_kv_heads);
  decode_mfma_shared_kernel<DT, D, S, kMfmaWaves>
      <<<grid, dim3(kMfmaWaves * 64), 0, stream>>>(grp, rest);
  return hipGetLastError();
}

// Whole groups sharing a prefix: final outputs, one workgroup per (group, kv head), head g on
// XCD g % 8 so a shared tile stays in one L2; each chunk picks its own cache policy.
template <Dt DT, int D, int S>
hipError_t launch_whole(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_units * (unsigned)p.num_kv_heads);
  decode_mfma_kernel<DT, D, S, kMfmaWaves, false, false, true, true>
      <<<grid, dim3(kMfmaWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

template <Dt DT, int D, int S>
hipError_t launch_s(bool partial, bool nt, const DecodeParams& p, hipStream_t stream) {
  if (p.group_members)
    return partial ? launch_grouped<DT, D, S>(p, stream) : launch_whole<DT, D, S>(p, stream);
  if (partial) return nt ? launch_p<DT, D, S, true, true>(p, stream) : launch_p<DT, D, S, true, false>(p, stream);
  return nt ? launch_p<DT, D, S, false, true>(p, stream) : launch_p<DT, D, S, false, false>(p, stream);
}

template <Dt DT, int S>
hipError_t launch_d(int head_dim, bool partial, bool nt, const DecodeParams& p,
                    hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_s<DT, 64, S>(partial, nt, p, stream);
    case 128: return launch_s<DT, 128, S>(partial, nt, p, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

template <int S>
hipError_t launch_decode_mfma_bs(Dt dt, int head_dim, bool partial, bool nt,
                                 const DecodeParams& p, hipStream_t stream) {
  switch (dt) {
    case Dt::F16: return launch_d<Dt::F16, S>(head_dim, partial, nt, p, stream);
    case Dt::BF16: return launch_d<Dt::BF16, S>(head_dim, partial, nt, p, stream);
    default: return hipErrorNotSupported;
  }
}

template <int S>
hipError_t launch_decode_mfma_shared_bs(Dt dt, int head_dim, const DecodeParams& grp,
                                        const DecodeParams& rest, hipStream_t stream) {
  switch (dt) {
    case Dt::F16:
      return head_dim == 64 ? launch_combined<Dt::F16, 64, S>(grp, rest, stream)
             : head_dim == 128 ? launch_combined<Dt::F16, 128, S>(grp, rest, stream)
                               : hipErrorNotSupported;
    case Dt::BF16:
      return head_dim == 64 ? launch_combined<Dt::BF16, 64, S>(grp, rest, stream)
             : head_dim == 128 ? launch_combined<Dt::BF16, 128, S>(grp, rest, stream)
                               : hipErrorNotSupported;
    default: return hipErrorNotSupported;
  }
}

template hipError_t launch_decode_mfma_bs<PKV_BLOCK_SIZE>(Dt, int, bool, bool,
                                                          const DecodeParams&, hipStream_t);
template hipError_t launch_decode_mfma_shared_bs<PKV_BLOCK_SIZE>(Dt, int, const DecodeParams&,
                                                                 const DecodeParams&,
                                                                 hipStream_t);

}  // namespace pkv
