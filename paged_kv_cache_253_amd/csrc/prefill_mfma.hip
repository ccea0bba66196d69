// Attention of several new query tokens per sequence over the paged cache,
// on the matrix cores: chunked prefill ("vLLM & High-Throughput Serving",
// section 4: a long prompt fed in chunks next to the decodes) and
// speculative verification ("AI Inference Serving at Scale", section 7:
// the target model scores K drafted tokens in one pass).  Sequence b's
// query tokens are its last Q_b cached tokens; the one at position p
// attends to cached tokens 0..p.
//
// The MFMA columns are (query token, query head) pairs: 16 * NT columns,
// i.e. 16 * NT / G query tokens of the group's G heads, in NT column tiles
// of 16 (a query tile).  Each 32-token step uses its K and V for every
// column tile:
//
//   S^T = K Q^T     2 * (head_dim / 32) * NT MFMAs (rows = tokens)
//   causal mask     token t is kept for a column iff t <= its position
//   online softmax  per column, in the result registers (as the decode)
//   O^T += V^T P^T  (head_dim / 16) * NT MFMAs
//
// One wavefront owns (context partition, KV head, sequence, query tile); the
// per-step work lives in Columns, on the decode's operand layouts
// (pa_mfma.hpp).
//
// The grid keeps all work of one (sequence, KV head) on one XCD, partition
// by partition, so the tiles that walk the same K/V at about the same pace
// find each other's data in that XCD's L2 (workgroups go to the XCDs
// round-robin by id).  A tile's context ends at its last query token, so
// later tiles of a long chunk read more of the cache than earlier ones.
#include "prefill_common.hpp"

namespace pa {
namespace {

using namespace prefill;

// ---------------------------------------------------------------------------
// One wavefront per query tile
// ---------------------------------------------------------------------------

template <int CK, int D, int BS, int NT>
__global__ __launch_bounds__(64) void prefill_mfma(const PrefillArgs args) {
  constexpr bool FP8 = one_byte<CK>();
  using C = Cfg<CK, D, BS>;
  const DecodeArgs& a = args.d;
  const Item it = locate_item(a, args.tiles);
  if (!it.ok) return;
  const int b = it.b, h = it.h, part = it.part;
  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const TileRange tr = tile_range(args, b, it.sub, part, 16 * NT / a.group);
  if (tr.i0 >= tr.nq) return;
  // no row of the tile reaches this partition (one that only the table
  // row's end empties still leaves its empty state for the merge)
  if (a.partition > 0 && tr.t0 >= tr.need) return;
  const int t0 = tr.t0, t1 = tr.t1;

  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (FP8) { kscale = a.k_scale[h]; vscale = a.v_scale[h]; }
  const float c2 = log2_factor(a.scale, kscale);  // q.k -> log2 units
  Columns<CK, D, BS, NT> cols;
  cols.init(a, tr.r0, tr.i0, tr.i1, tr.first_pos, h, col, grp, c2);

  if (t0 < t1) {
    const LaneOffsets<CK, D, BS> lo(grp, col);
    const char* kc = reinterpret_cast<const char*>(a.k_cache);
    const char* vc = reinterpret_cast<const char*>(a.v_cache);
    const int32_t* table = a.block_tables + (size_t)b * a.max_blocks;
    const int nsteps = (t1 - t0 + kStep - 1) / kStep;
    const int lb_first = t0 / BS;
    const int lb_last = (t1 - 1) / BS;
    int chunk_base = lb_first;
    int tbl = (chunk_base + lane <= lb_last) ? table[chunk_base + lane] : 0;
    auto phys_of = [&](int lb) -> int64_t {
      int p = readlane(tbl, lb - chunk_base);
      return (p < 0 || (int64_t)p >= a.num_blocks) ? 0 : (int64_t)p;
    };
    auto issue = [&](StepBuf<CK, D, BS>& sb, int step) {
      const int lb0 = (t0 + step * kStep) / BS;
      const int lb1 = min(lb0 + C::kBlocksPerStep - 1, lb_last);
      if (lb1 - chunk_base >= 64) {  // slide the table window
        chunk_base = lb0;
        tbl = (chunk_base + lane <= lb_last) ? table[chunk_base + lane] : 0;
      }
      const int64_t p0 = phys_of(lb0);
      const int64_t p1 = (C::kBlocksPerStep == 2) ? phys_of(lb1) : p0;
      load_step(sb, kc, vc, (p0 * a.num_kv_heads + h) * C::kTile, (p1 * a.num_kv_heads + h) * C::kTile,
                lo, grp);
    };
    StepBuf<CK, D, BS> bufA, bufB;
    issue(bufA, 0);
    for (int step = 0; step < nsteps; step += 2) {
      issue(bufB, min(step + 1, nsteps - 1));
      cols.step(bufA, t0 + step * kStep, t1, grp, c2);
      if (step + 1 >= nsteps) break;
      issue(bufA, min(step + 2, nsteps - 1));
      cols.step(bufB, t0 + (step + 1) * kStep, t1, grp, c2);
    }
  }
  cols.finish(a, part, grp, c2, vscale);
}

template <int CK, int D, int BS, int NT>
hipError_t launch_nt(const PrefillArgs& p, hipStream_t stream) {
  constexpr bool FP8 = one_byte<CK>();
  const DecodeArgs& a = p.d;
  const Elem e = CK == kI4 ? Elem::I4 : (FP8 ? Elem::FP8 : Elem::BF16);  // FP8 kinds alike
  const int tiles = prefill_query_tiles(a.group, p.max_query_len, prefill_max_column_tiles(e, D));
  const int parts = a.partition ? a.max_parts : 1;
  const long long pairs = (long long)a.num_seqs * a.num_kv_heads;
  const long long groups = (pairs + kXcds - 1) / kXcds * kXcds * parts * tiles;
  if (groups > INT32_MAX) return hipErrorInvalidValue;
  PrefillArgs q = p;
  q.tiles = tiles;
  hipLaunchKernelGGL((prefill_mfma<CK, D, BS, NT>), dim3((unsigned)groups), dim3(64), 0, stream, q);
  return hipGetLastError();
}

template <int CK, int D, int BS>
hipError_t launch_shape(const PrefillArgs& p, hipStream_t stream) {
  constexpr int kMaxNT = (!one_byte<CK>() && D == 128) ? 2 : 4;  // as prefill_max_column_tiles
  switch (prefill_column_tiles(p.d.group, p.max_query_len, kMaxNT)) {
    case 1: return launch_nt<CK, D, BS, 1>(p, stream);
    case 2: return launch_nt<CK, D, BS, 2>(p, stream);
    default:
      if constexpr (kMaxNT >= 4) return launch_nt<CK, D, BS, 4>(p, stream);
      return hipErrorInvalidValue;
  }
}

template <int CK>
hipError_t dispatch(const PrefillArgs& p, int head_dim, int block_size, hipStream_t s) {
  if (head_dim == 128 && block_size == 16) return launch_shape<CK, 128, 16>(p, s);
  if (head_dim == 128 && block_size == 32) return launch_shape<CK, 128, 32>(p, s);
  if (head_dim == 64 && block_size == 16) return launch_shape<CK, 64, 16>(p, s);
  if (head_dim == 64 && block_size == 32) return launch_shape<CK, 64, 32>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& p, Elem cache, int head_dim, int block_size,
                               hipStream_t stream) {
  if (prefill_uses_lds(cache, p.d.group, p.max_query_len))
    return launch_prefill_lds(p, head_dim, block_size, stream);
  if (cache == Elem::BF16) return dispatch<kBF16>(p, head_dim, block_size, stream);
  if (cache == Elem::FP8) return dispatch<kE4M3>(p, head_dim, block_size, stream);
  if (cache == Elem::E5M2) return dispatch<kE5M2>(p, head_dim, block_size, stream);
  if (cache == Elem::I4) return dispatch<kI4>(p, head_dim, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa

