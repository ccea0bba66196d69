// Chunked prefill with long query runs ("vLLM & High-Throughput Serving",
// section 4): the wavefronts of a workgroup share each 32-token step's K
// and V tiles through LDS (the per-column work is that of prefill_mfma.hip,
// prefill_common.hpp).  Eight wavefronts of two column tiles per
// workgroup, one workgroup per CU, a barrier every four steps (measured on
// MI355X, chunked prefill at 8K context: 604 us, against 620 us for a
// barrier every two steps and 647 us for four wavefronts per workgroup at
// two workgroups per CU; a barrier every step 804 us against 750 us for
// every two steps at the time, the block-table reads
// of a step's pieces at their issue 721 us against 704 us read a step
// ahead; earlier revisions: eight wavefronts per workgroup 967 against
// 948 us, four column tiles per wavefront with the accumulators in AGPRs
// 1,416 us, one column tile per wavefront at three workgroups per CU 1,008
// against 802 us, one wavefront per query tile without LDS sharing
// 1,105 us).
#include "prefill_common.hpp"

namespace pa {
namespace {

using namespace prefill;

// ---------------------------------------------------------------------------
// Long query runs (chunked prefill): one workgroup of W wavefronts per query
// block of W query tiles, sharing each step's K and V through LDS
// ---------------------------------------------------------------------------
// With one wavefront per query tile every tile streams the whole context
// through its own registers: each 16 KiB bf16 step feeds only 32 MFMA
// columns, and the L2 delivers the same tiles once per query tile.  Here
// the W wavefronts of a workgroup take consecutive query tiles of one
// (sequence, KV head); each step's tiles are read from memory once, by all
// lanes of the workgroup (one 16-byte piece each), written to LDS, and
// every wavefront builds its MFMA operands from LDS in the register layout
// the streaming loads give (so the QK, softmax and PV code is the one
// above).  Each lane loads its pieces of a step into one of two register
// sets and writes them to one of eight LDS step buffers two steps later,
// after computing the step before; a barrier every four steps makes the
// four steps just written visible and frees the four just read (8 x 18 KiB
// per workgroup).
//
// LDS layout (one buffer): K as [token group m][chunk][16 tokens] of 16-byte
// pieces (chunk = 8 head dimensions), i.e. operand k[m][j] of lane (grp,
// col) at [m][grp + 4 j][col]; V as [dimension][32 tokens] bf16 rows padded
// to 40 elements (80 bytes: the 16 lanes of a lane group read 16 rows
// without bank conflicts), operand v[dt] of lane (grp, col) at
// [16 dt + col][8 grp].

template <int D>
struct LdsStep {
  u32x4 k[2][D / 8][16];
  __bf16 v[D][40];
};

template <int CK, int D, int BS, int NT, int W>
__global__ __launch_bounds__(64 * W) void prefill_lds(const PrefillArgs args) {
  static_assert(CK == kBF16, "the LDS-shared prefill takes bf16 caches");
  using C = Cfg<CK, D, BS>;
  constexpr int kThreads = 64 * W;
  constexpr int kPieces = 2 * (D / 8) * 16;  // 16-byte pieces of K (and of V) per step
  const DecodeArgs& a = args.d;
  const Item it = locate_item(a, args.tiles);
  if (!it.ok) return;  // the whole workgroup: uniform
  const int b = it.b, h = it.h, part = it.part;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int rows_w = 16 * NT / a.group;  // query rows of one wavefront
  const TileRange tr = tile_range(args, b, it.sub, part, rows_w * W);
  if (tr.i0 >= tr.nq) return;
  if (a.partition > 0 && tr.t0 >= tr.need) return;
  const int t0 = tr.t0, t1 = tr.t1;

  // this wavefront's rows of the block (none for a wavefront past its end)
  const int wi0 = tr.i0 + wave * rows_w;
  const int wi1 = min(wi0 + rows_w, tr.i1);
  const bool mine = wi0 < wi1;
  const float c2 = a.scale * kLog2e;
  Columns<CK, D, BS, NT> cols;
  if (mine) cols.init(a, tr.r0, wi0, wi1, tr.first_pos, h, col, grp, c2);
  // last token any of this wavefront's rows sees
  const int wlast = mine ? min(tr.first_pos + wi1 - 1, t1 - 1) : -1;

  __shared__ LdsStep<D> lds[8];
  if (t0 < t1) {
    const char* kc = reinterpret_cast<const char*>(a.k_cache);
    const char* vc = reinterpret_cast<const char*>(a.v_cache);
    // block-table entries through the constant address space: scalar loads,
    // whatever the kernel does before them
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    const const_i32 table = (const_i32)a.block_tables + (size_t)b * a.max_blocks;
    const int nsteps = (t1 - t0 + kStep - 1) / kStep;
    const int lb_last = (t1 - 1) / BS;
    constexpr int kPer = (kPieces + kThreads - 1) / kThreads;  // pieces per lane and tensor
    struct Pieces { u32x4 k[kPer], v[kPer]; };
    Pieces set0, set1;
    auto tile_of = [&](int lb) -> int64_t {
      int p = table[lb];
      p = (p < 0 || (int64_t)p >= a.num_blocks) ? 0 : p;
      return ((int64_t)p * a.num_kv_heads + h) * C::kTile;
    };
    // the tiles of step `step` (table entries read with scalar loads, ahead
    // of their use: a wait on them also waits on the LDS operations in
    // flight)
    struct Tiles { int64_t t0, t1; };
    auto locate = [&](int step) -> Tiles {
      const int lb0 = (t0 + step * kStep) / BS;
      const int64_t tile0 = tile_of(lb0);
      return {tile0, C::kBlocksPerStep == 2 ? tile_of(min(lb0 + 1, lb_last)) : tile0};
    };
    // the pieces of a step this lane carries: K piece (m, chunk, token), V
    // piece (dimension, 8-token group)
    auto fetch = [&](Pieces& ps, const Tiles& tl) {
      const int64_t tile0 = tl.t0, tile1 = tl.t1;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int pc = tid + i * kThreads;
        if (pc < kPieces) {
          const int m = pc / (kPieces / 2), chunk = (pc / 16) % (D / 8), tok = pc % 16;
          const int64_t ko = BS == 16 ? (m ? tile1 : tile0) + (chunk * 16 + tok) * 16
                                      : tile0 + (chunk * 32 + 16 * m + tok) * 16;
          ps.k[i] = stream_load<u32x4>(kc + ko);
          // tokens 8 g8 .. + 7 of dimension dim; 16 consecutive lanes take 16
          // dimensions of one token group, so their LDS writes (80-byte rows)
          // fall in distinct banks
          const int dim = pc % 16 + 16 * (pc / 64), g8 = (pc / 16) % 4;
          const int64_t vo = BS == 16 ? ((g8 >> 1) ? tile1 : tile0) + dim * 32 + (g8 & 1) * 16
                                      : tile0 + dim * 64 + g8 * 16;
          ps.v[i] = stream_load<u32x4>(vc + vo);
        }
      }
    };
    auto store = [&](const Pieces& ps, LdsStep<D>& L) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int pc = tid + i * kThreads;
        if (pc < kPieces) {
          const int m = pc / (kPieces / 2), chunk = (pc / 16) % (D / 8), tok = pc % 16;
          L.k[m][chunk][tok] = ps.k[i];
          const int dim = pc % 16 + 16 * (pc / 64), g8 = (pc / 16) % 4;
          *reinterpret_cast<u32x4*>(&L.v[dim][8 * g8]) = ps.v[i];
        }
      }
    };
    StepBuf<CK, D, BS> sb;
    auto compute = [&](const LdsStep<D>& L, int step) {
      const int base = t0 + step * kStep;
      if (mine && base <= wlast) {  // a step no row of this wavefront reaches is skipped
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < C::kKLoads; ++j) sb.k[m][j] = L.k[m][grp + 4 * j][col];
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt)
          sb.v[dt].w = *reinterpret_cast<const u32x4*>(&L.v[16 * dt + col][8 * grp]);
        cols.step(sb, base, t1, grp, c2);
      }
    };
    // step n's pieces travel in set n % 2 and LDS buffer n % 8; a barrier
    // every four steps
    fetch(set0, locate(0));
    if (nsteps > 1) fetch(set1, locate(1));
    store(set0, lds[0]);
    if (nsteps > 1) store(set1, lds[1]);
    if (nsteps > 2) fetch(set0, locate(2));
    if (nsteps > 3) fetch(set1, locate(3));
    if (nsteps > 2) store(set0, lds[2]);
    if (nsteps > 3) store(set1, lds[3]);
    if (nsteps > 4) fetch(set0, locate(4));
    if (nsteps > 5) fetch(set1, locate(5));
    __syncthreads();
    // four steps per barrier, unrolled twice so that every LDS buffer index
    // is a constant
    auto four_steps = [&](int step, LdsStep<D>& c0, LdsStep<D>& c1, LdsStep<D>& c2_, LdsStep<D>& c3,
                          LdsStep<D>& w0, LdsStep<D>& w1, LdsStep<D>& w2, LdsStep<D>& w3) {
      const Tiles n0 = step + 6 < nsteps ? locate(step + 6) : Tiles{0, 0};
      const Tiles n1 = step + 7 < nsteps ? locate(step + 7) : Tiles{0, 0};
      const Tiles n2 = step + 8 < nsteps ? locate(step + 8) : Tiles{0, 0};
      const Tiles n3 = step + 9 < nsteps ? locate(step + 9) : Tiles{0, 0};
      compute(c0, step);
      if (step + 4 < nsteps) store(set0, w0);
      if (step + 6 < nsteps) fetch(set0, n0);
      if (step + 1 < nsteps) compute(c1, step + 1);
      if (step + 5 < nsteps) store(set1, w1);
      if (step + 7 < nsteps) fetch(set1, n1);
      if (step + 2 < nsteps) compute(c2_, step + 2);
      if (step + 6 < nsteps) store(set0, w2);
      if (step + 8 < nsteps) fetch(set0, n2);
      if (step + 3 < nsteps) compute(c3, step + 3);
      if (step + 7 < nsteps) store(set1, w3);
      if (step + 9 < nsteps) fetch(set1, n3);
      __syncthreads();
    };
    for (int step = 0; step < nsteps; step += 8) {
      four_steps(step, lds[0], lds[1], lds[2], lds[3], lds[4], lds[5], lds[6], lds[7]);
      if (step + 4 >= nsteps) break;
      four_steps(step + 4, lds[4], lds[5], lds[6], lds[7], lds[0], lds[1], lds[2], lds[3]);
    }
  }
  if (mine) cols.finish(a, part, grp, c2, 1.0f);
}

// Query rows per workgroup of the LDS-shared prefill, and whether a launch
// takes it: bf16 cache with query runs long enough to fill a workgroup.
// Eight wavefronts of two column tiles per workgroup, one workgroup per CU
// (230 VGPRs: two wavefronts per SIMD; 144 KiB of LDS).
constexpr int kLdsWaves = 8;
constexpr int kLdsNT = 2;

template <int D, int BS>
hipError_t launch_lds(const PrefillArgs& p, hipStream_t stream) {
  const DecodeArgs& a = p.d;
  const int rows = 16 * kLdsNT * kLdsWaves / a.group;
  const int tiles = (p.max_query_len + rows - 1) / rows;
  const int parts = a.partition ? a.max_parts : 1;
  const long long pairs = (long long)a.num_seqs * a.num_kv_heads;
  const long long groups = (pairs + kXcds - 1) / kXcds * kXcds * parts * tiles;
  if (groups > INT32_MAX) return hipErrorInvalidValue;
  PrefillArgs q = p;
  q.tiles = tiles;
  hipLaunchKernelGGL((prefill_lds<kBF16, D, BS, kLdsNT, kLdsWaves>), dim3((unsigned)groups),
                     dim3(64 * kLdsWaves), 0, stream, q);
  return hipGetLastError();
}

}  // namespace

bool prefill_uses_lds(Elem cache, int group, int max_query_len) {
  return cache == Elem::BF16 &&
         (long long)group * max_query_len >= 16 * kLdsNT * kLdsWaves;
}

hipError_t launch_prefill_lds(const PrefillArgs& p, int head_dim, int block_size, hipStream_t stream) {
  if (head_dim == 128 && block_size == 16) return launch_lds<128, 16>(p, stream);
  if (head_dim == 128 && block_size == 32) return launch_lds<128, 32>(p, stream);
  if (head_dim == 64 && block_size == 16) return launch_lds<64, 16>(p, stream);
  if (head_dim == 64 && block_size == 32) return launch_lds<64, 32>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
