// Paged decode attention on the vector ALUs (fp32, and fp16/bf16 when the query group is too
// small for a dense product). One workgroup of NW waves owns one (sequence, range) unit for
// HPW adjacent kv heads (two when the kv head count is even, so the two tiles of a block it
// reads at once are one contiguous run); each of a head's NW / HPW waves walks every
// (NW / HPW)-th step of the range with an online softmax, and a head's waves merge their
// (max, sum, accumulator) states through LDS at the end.
//
// The operation is attention over non-contiguous KV-cache blocks (vAttention, section 3.1
// "Requires re-writing the attention kernel"): each block is found through the sequence's
// block table (Qualiteg, "About PagedAttention for LLM serving", "There are logical blocks
// and physical blocks, and the two are linked by a block table"), and each sequence uses
// only its own length, with no padding (same post, item 2-1).
//
// A wave steps through the range CS = min(S, 32) positions at a time: a whole block up to
// 32 positions, else a 32-position slice of one (so registers do not grow with S).
// Lane geometry for the CS rows of a K tile [S][D] of a (block, kv head): a token row is LPR
// lanes x 16 bytes, so one wave load covers ROWS = 64 / LPR rows; lane (r, c) with
// r = lane / LPR and c = lane % LPR owns positions r*TPL .. r*TPL+TPL-1 of every step and the
// 16-byte column piece c of the K row. A block stores V in column groups of CS positions, each
// a [D][CS] tile, so a step reads one group; the same lane reads, for each of its VEC head-dim
// rows d = c + LPR*y, the TPL contiguous positions it owns; so the softmax weights a lane
// needs for P.V are the ones it computed itself, with no exchange.
#include "kernels.hpp"

#ifndef PKV_BLOCK_SIZE
#error "build once per block size with -DPKV_BLOCK_SIZE=16|32|64|128|256"
#endif

namespace pkv {
namespace {

template <Dt DT, int D, int S, int G, int NW, int HPW, bool PARTIAL, bool NTL>
__global__ void __launch_bounds__(NW * 64)
decode_valu_kernel(const DecodeParams a) {
  constexpr int WPH = NW / HPW;  // waves per kv head
  static_assert(WPH * HPW == NW, "waves must split evenly over the workgroup's kv heads");
  constexpr int EB = Elt<DT>::bytes;
  constexpr int VEC = 16 / EB;   // elements per 16-byte piece
  constexpr int LPR = D / VEC;   // lanes per K row
  constexpr int ROWS = 64 / LPR; // K rows per wave load
  constexpr int CS = S < 32 ? S : 32;  // positions per step
  constexpr int SPB = S / CS;    // steps per block
  constexpr int TPL = CS / ROWS; // positions per lane per step
  constexpr int VB = TPL * EB;   // bytes per lane per V^T row
  constexpr int VW = VB / 4;     // 32-bit words per lane per V^T row
  static_assert(LPR >= 8 && LPR <= 32 && TPL >= 1, "unsupported head_dim/block_size/dtype");
  using T = typename Elt<DT>::T;

  __shared__ float sh_m[NW][G];
  __shared__ float sh_l[NW][G];
  __shared__ float sh_acc[NW][G][D];
  __shared__ float sh_new[HPW][G];
  __shared__ float sh_vnew[HPW][D];

  const int Hkv = a.num_kv_heads;
  const int H = a.num_heads;
  const int MB = a.max_blocks_per_seq;
  // A workgroup takes kv heads HPW gg .. HPW gg + HPW - 1 (head group gg; waves 0 .. WPH-1
  // the first head). Workgroups go to the XCDs round robin (w % 8). Unshared KV (non-temporal
  // loads): every head group of a unit on one XCD (groups of 8 HG workgroups hold 8 units,
  // head group gg of the group's unit j at 8 gg + j), so an XCD streams whole blocks of its
  // sequences. Cached loads (shared prefix blocks): head group gg of every unit on XCD gg % 8,
  // so a shared tile stays in one L2.
  const int w = blockIdx.x;
  const int HG = Hkv / HPW;  // kv-head groups per unit
  const int lane = lane_id();
  const int wave = wave_id();
  const int hw = wave / WPH;  // this wave's head within the workgroup
  const int wv = wave % WPH;  // this wave's index among its head's waves
  int g, slot;
  if constexpr (NTL) {
    constexpr int XC = 8;
    g = (w % (XC * HG)) / XC;
    slot = (w / (XC * HG)) * XC + w % XC;
    if (slot >= a.num_units) return;  // the grid is padded to whole groups of 8 units
  } else {
    g = w % HG;
    slot = w / HG;
  }
  g = g * HPW + hw;
  int unit = a.work_items ? a.work_items[slot] : slot;
  unit = min(max(unit, 0), a.num_seqs * a.num_ranges - 1);
  const int part = unit % a.num_ranges;
  const int i = unit / a.num_ranges;
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int32_t* bt = a.block_tables + (size_t)i * MB;
  auto table = [&](int j) { return bt[j]; };
  const int start = part * a.range_tokens;

  // A head's waves take steps start/CS + wv, + WPH, ... (step b covers positions b*CS ..
  // b*CS+CS-1 of logical block b / SPB); the first one's id is fetched before the context
  // length arrives (any entry of the row may be read; ids are clamped before use).
  const int b_first = start / CS + wv;
  const int first_id = b_first / SPB < MB ? table(b_first / SPB) : 0;

  int L = a.context_lens[i];
  L = min(max(L, 0), MB * S);
  if (start >= L) {
    if (!PARTIAL && part == 0) {
      T* o = reinterpret_cast<T*>(a.out) + ((size_t)i * H + (size_t)(g - hw) * G) * D;
      for (int e = threadIdx.x; e < HPW * G * D; e += NW * 64) o[e] = from_f32<DT>(0.0f);
    }
    return;
  }
  // With a fused write, position L-1 comes from new_key/new_value (this is then the sequence's
  // last range) and the cache is read only up to L-2.
  const bool fused = a.new_key != nullptr && start + a.range_tokens >= L;
  const int end = min(start + a.range_tokens, L) - (fused ? 1 : 0);
  const int blk_hi = (end + CS - 1) / CS;  // first step past the cached range

  // This lane's 16-byte piece of q for every head of the group, widened to fp32.
  float qf[G][VEC];
  {
    const char* qb = reinterpret_cast<const char*>(a.q) +
                     ((size_t)i * H + (size_t)g * G) * D * EB + (size_t)c * 16;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qb + (size_t)h * D * EB);
      const uint32_t wq[4] = {v.x, v.y, v.z, v.w};
      unpack_words<DT, 4>(wq, qf[h]);
    }
  }

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int y = 0; y < VEC; ++y) acc[h][y] = 0.0f;
  }

  const size_t tile_bytes = (size_t)S * D * EB;
  const size_t id_stride = (size_t)Hkv * tile_bytes;
  const char* kpool = reinterpret_cast<const char*>(a.k_cache) + (size_t)g * tile_bytes;
  const char* vpool = reinterpret_cast<const char*>(a.v_cache) + (size_t)g * tile_bytes;
  const int k_off = (r * TPL) * D * EB + c * 16;   // + x * D * EB
  const int v_off = c * CS * EB + r * TPL * EB;    // + y * LPR * CS * EB

  struct Regs {
    uint32_t k[TPL][4];
    uint32_t v[VEC][VW];
  };

  auto clamp_id = [&](int id) { return min(max(id, 0), a.num_blocks - 1); };
  auto load = [&](int id, int b, Regs& R) {
    const int ob = (b % SPB) * CS;  // first position of step b within its block
    const char* kt = kpool + (size_t)id * id_stride + (size_t)ob * D * EB + k_off;
    const char* vt = vpool + (size_t)id * id_stride + (size_t)ob * D * EB + v_off;
#pragma unroll
    for (int x = 0; x < TPL; ++x) load_words<16, NTL>(kt + x * D * EB, R.k[x]);
#pragma unroll
    for (int y = 0; y < VEC; ++y) load_words<VB, NTL>(vt + y * LPR * CS * EB, R.v[y]);
  };

  auto compute = [&](int b, const Regs& R) {
    float s[TPL][G];
#pragma unroll
    for (int x = 0; x < TPL; ++x) {
      float kf[VEC];
      unpack_words<DT, 4>(R.k[x], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) t = fmaf(qf[h][e], kf[e], t);
        s[x][h] = t;
      }
    }
#pragma unroll
    for (int x = 0; x < TPL; ++x)
#pragma unroll
      for (int h = 0; h < G; ++h) s[x][h] = group_reduce<LPR>(s[x][h], OpAdd());

    const int pos0 = b * CS + r * TPL;
    float mx[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = -INFINITY;
#pragma unroll
      for (int x = 0; x < TPL; ++x) {
        s[x][h] = (pos0 + x < end) ? s[x][h] * a.scale_log2e : -INFINITY;
        mx[h] = fmaxf(mx[h], s[x][h]);
      }
      mx[h] = cross_group_reduce<LPR>(mx[h], OpMax());
      const float mnew = fmaxf(m[h], mx[h]);
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mnew);
      m[h] = mnew;
      l[h] *= alpha;
#pragma unroll
      for (int y = 0; y < VEC; ++y) acc[h][y] *= alpha;
#pragma unroll
      for (int x = 0; x < TPL; ++x) {
        s[x][h] = __builtin_amdgcn_exp2f(s[x][h] - mnew);
        l[h] += s[x][h];
      }
    }
    const bool tail = (b + 1) * CS > end;
#pragma unroll
    for (int y = 0; y < VEC; ++y) {
      float vf[TPL];
      unpack_words<DT, VW>(R.v[y], vf);
      if (tail) {
#pragma unroll
        for (int x = 0; x < TPL; ++x) vf[x] = (pos0 + x < end) ? vf[x] : 0.0f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int x = 0; x < TPL; ++x) acc[h][y] = fmaf(s[x][h], vf[x], acc[h][y]);
    }
  };

  // Position L-1 joins the merge below as one more partial state (m = its logit, l = 1,
  // acc = its V row). Its rows are loaded before the first block (vector loads return in
  // order, so waiting for them below does not wait for the block).
  const char* kn = reinterpret_cast<const char*>(a.new_key) + ((size_t)i * Hkv + g) * D * EB;
  const T* vn = reinterpret_cast<const T*>(a.new_value) + ((size_t)i * Hkv + g) * D;
  u32x4 kpiece = {0u, 0u, 0u, 0u};
  u32x4 krow = {0u, 0u, 0u, 0u};
  T vrow[D / 64];
  int slot_blk = 0;
  if (fused) {
    if (wv == WPH - 1) kpiece = *reinterpret_cast<const u32x4*>(kn + (size_t)c * 16);
    if (wv == 0) {
      slot_blk = table((L - 1) / S);
      if (lane < D * EB / 16) krow = reinterpret_cast<const u32x4*>(kn)[lane];
#pragma unroll
      for (int e = 0; e < D / 64; ++e) vrow[e] = vn[lane + 64 * e];
    }
  }

  // Consumes the new rows loaded above (after this wave's first loads are in flight): the
  // head's last wave's logits and its first wave's LDS copy of the V row.
  auto use_new_rows = [&]() {
    if (wv == WPH - 1) {
      const uint32_t kw4[4] = {kpiece.x, kpiece.y, kpiece.z, kpiece.w};
      float kf[VEC];
      unpack_words<DT, 4>(kw4, kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) t = fmaf(qf[h][e], kf[e], t);
        t = group_reduce<LPR>(t, OpAdd());
        if (lane == 0) sh_new[hw][h] = t * a.scale_log2e;
      }
    }
    if (wv == 0) {
#pragma unroll
      for (int e = 0; e < D / 64; ++e) {
        const int d = lane + 64 * e;
        if constexpr (DT == Dt::F32) sh_vnew[hw][d] = vrow[e];
        else if constexpr (DT == Dt::BF16) sh_vnew[hw][d] = bits_f((uint32_t)vrow[e] << 16);
        else sh_vnew[hw][d] = (float)vrow[e];
      }
    }
  };

  int b = b_first;
  if (b < blk_hi) {
    Regs A, B;
    load(clamp_id(first_id), b, A);
    int id = b + WPH < blk_hi ? clamp_id(table((b + WPH) / SPB)) : 0;
    if (fused) use_new_rows();
    // Two register sets: step b + WPH loads while step b computes; its id was fetched one
    // step earlier still.
    while (true) {
      if (b + WPH < blk_hi) {
        load(id, b + WPH, B);
        if (b + 2 * WPH < blk_hi) id = clamp_id(table((b + 2 * WPH) / SPB));
      }
      compute(b, A);
      b += WPH;
      if (b >= blk_hi) break;
      if (b + WPH < blk_hi) {
        load(id, b + WPH, A);
        if (b + 2 * WPH < blk_hi) id = clamp_id(table((b + 2 * WPH) / SPB));
      }
      compute(b, B);
      b += WPH;
      if (b >= blk_hi) break;
    }
  } else if (fused) {
    use_new_rows();
  }

  // The new rows go to the slot the table maps position L-1 to. The stores come after every
  // block-table read so the table can stay in the scalar cache (a store that might alias it
  // would force those reads through the vector memory path).
  if (fused && wv == 0) {
    const int p = L - 1;
    const size_t tile = ((size_t)clamp_id(slot_blk) * Hkv + g) * S * D;
    T* kc = reinterpret_cast<T*>(a.k_cache) + tile + (size_t)(p % S) * D;
    T* vc = reinterpret_cast<T*>(a.v_cache) + tile + (size_t)((p % S) / CS) * CS * D + p % CS;
    if (lane < D * EB / 16) reinterpret_cast<u32x4*>(kc)[lane] = krow;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) vc[(size_t)(lane + 64 * e) * CS] = vrow[e];
  }

  // Sum each lane's positions over the row groups (lanes that share c hold the same columns).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = cross_group_reduce<LPR>(l[h], OpAdd());
#pragma unroll
    for (int y = 0; y < VEC; ++y) acc[h][y] = cross_group_reduce<LPR>(acc[h][y], OpAdd());
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int y = 0; y < VEC; ++y) sh_acc[wave][h][c + LPR * y] = acc[h][y];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sh_m[wave][h] = m[h];
      sh_l[wave][h] = l[h];
    }
  }
  __syncthreads();

  // Merge each head's waves: M = max m_w, weights 2^(m_w - M) (a wave without blocks has
  // m = -inf).
  for (int e = threadIdx.x; e < HPW * G * D; e += NW * 64) {
    const int hh = e / (G * D);
    const int h = (e / D) % G;
    const int d = e % D;
    float M = fused ? sh_new[hh][h] : -INFINITY;
#pragma unroll
    for (int v = 0; v < WPH; ++v) M = fmaxf(M, sh_m[hh * WPH + v][h]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int v = 0; v < WPH; ++v) {
      const float f = __builtin_amdgcn_exp2f(sh_m[hh * WPH + v][h] - M);
      num = fmaf(f, sh_acc[hh * WPH + v][h][d], num);
      den = fmaf(f, sh_l[hh * WPH + v][h], den);
    }
    if (fused) {
      const float f = __builtin_amdgcn_exp2f(sh_new[hh][h] - M);
      num = fmaf(f, sh_vnew[hh][d], num);
      den += f;
    }
    const float o = num / den;
    const size_t row = (size_t)i * H + (size_t)(g - hw + hh) * G + h;
    if constexpr (PARTIAL) {
      const size_t rec = row * a.num_ranges + part;
      a.tmp_out[rec * D + d] = o;
      if (d == 0) {
        a.max_logits[rec] = M * kLn2;
        a.exp_sums[rec] = den;
      }
    } else {
      reinterpret_cast<T*>(a.out)[row * D + d] = from_f32<DT>(o);
    }
  }
}

constexpr int kValuWaves = 4;

template <Dt DT, int D, int S, int G, int HPW>
hipError_t launch_h(bool partial, bool nt, const DecodeParams& p, hipStream_t stream) {
  constexpr int NW = kValuWaves;
  const unsigned units = nt ? (p.num_units + 7) / 8 * 8 : p.num_units;
  const dim3 grid(units * (unsigned)(p.num_kv_heads / HPW));
  const dim3 block(NW * 64);
  if (partial) {
    if (nt) decode_valu_kernel<DT, D, S, G, NW, HPW, true, true><<<grid, block, 0, stream>>>(p);
    else decode_valu_kernel<DT, D, S, G, NW, HPW, true, false><<<grid, block, 0, stream>>>(p);
  } else {
    if (nt) decode_valu_kernel<DT, D, S, G, NW, HPW, false, true><<<grid, block, 0, stream>>>(p);
    else decode_valu_kernel<DT, D, S, G, NW, HPW, false, false><<<grid, block, 0, stream>>>(p);
  }
  return hipGetLastError();
}

template <Dt DT, int D, int S, int G>
hipError_t launch_g(bool partial, bool nt, const DecodeParams& p, hipStream_t stream) {
  if (p.num_kv_heads % 2 == 0)
    return launch_h<DT, D, S, G, 2>(partial, nt, p, stream);
  return launch_h<DT, D, S, G, 1>(partial, nt, p, stream);
}

template <Dt DT, int D, int S>
hipError_t launch_s(int group, bool partial, bool nt, const DecodeParams& p,
                    hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<DT, D, S, 1>(partial, nt, p, stream);
    case 2: return launch_g<DT, D, S, 2>(partial, nt, p, stream);
    case 4: return launch_g<DT, D, S, 4>(partial, nt, p, stream);
    case 8: return launch_g<DT, D, S, 8>(partial, nt, p, stream);
    default: return hipErrorNotSupported;
  }
}

template <Dt DT, int S>
hipError_t launch_d(int head_dim, int group, bool partial, bool nt, const DecodeParams& p,
                    hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_s<DT, 64, S>(group, partial, nt, p, stream);
    case 128: return launch_s<DT, 128, S>(group, partial, nt, p, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

template <int S>
hipError_t launch_decode_valu_bs(Dt dt, int head_dim, int group, bool partial, bool nt,
                                 const DecodeParams& p, hipStream_t stream) {
  switch (dt) {
    case Dt::F32: return launch_d<Dt::F32, S>(head_dim, group, partial, nt, p, stream);
    case Dt::F16: return launch_d<Dt::F16, S>(head_dim, group, partial, nt, p, stream);
    case Dt::BF16: return launch_d<Dt::BF16, S>(head_dim, group, partial, nt, p, stream);
  }
  return hipErrorNotSupported;
}

template hipError_t launch_decode_valu_bs<PKV_BLOCK_SIZE>(Dt, int, int, bool, bool,
                                                          const DecodeParams&, hipStream_t);

}  // namespace pkv
