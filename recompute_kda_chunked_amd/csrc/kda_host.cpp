// Host side of the C ABI declared in include/kda.h: validation, planning of
// chunks and streaming segments, workspace carving and kernel launches.
//
// Recompute policy ("KDA Memory with Recompute: FLA vs cuDNN Frontend
// FROST", sections "Both sides really use recomputation" and "Takeaway"):
// the forward keeps nothing for the backward. The backward rebuilds every
// intermediate from the inputs, one segment of chunks at a time, from the
// last segment to the first, so the workspace is bounded by the segment size
// rather than by the sequence length:
//   checkpoint pass  chunk-local + state scan over segments 0..S-2, keeping
//                    only the state that enters each segment
//   per segment      chunk-local (recompute w, u, qg, kg, Aqk, T)
//                    state scan from the segment's checkpoint (records h, Vn)
//                    reverse state-gradient scan (records dh', dVn)
//                    token-parallel gradients (final dtype, written once)
//   finally          fixed-order reduction of the gate-parameter partials
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

using namespace kda;

namespace {

thread_local char g_msg[256];

// Largest |L| (gate_lower_bound) for which every gate factor the kernels form
// stays finite in fp32: 15 * 5.9 = 88.5 < ln(FLT_MAX) = 88.72.
constexpr float kMaxGateBound = 5.9f;

bool supported(int dtype, int D, int C) {
  if (dtype == KDA_F32)
    return (D == 64 && (C == 16 || C == 32 || C == 64)) || (D == 128 && (C == 16 || C == 32));
  if (dtype == KDA_BF16) return (D == 64 || D == 128) && (C == 32 || C == 64);
  return false;
}

int check_problem(const kda_problem* p) {
  if (!p || !p->cu_seqlens_host) return KDA_ERR_INVALID;
  if (p->n_seqs < 1 || p->H < 1 || p->K < 1 || p->V < 1 || p->total_tokens < 1)
    return KDA_ERR_INVALID;
  if (p->total_tokens > 0x7fffffffLL) return KDA_ERR_INVALID;
  const int32_t* cu = p->cu_seqlens_host;
  if (cu[0] != 0) return KDA_ERR_INVALID;
  for (int n = 0; n < p->n_seqs; ++n)
    if (cu[n + 1] < cu[n]) return KDA_ERR_INVALID;
  if (cu[p->n_seqs] != p->total_tokens) return KDA_ERR_INVALID;
  if (!(p->gate_lower_bound < 0.f) || !std::isfinite(p->gate_lower_bound)) return KDA_ERR_INVALID;
  // The gated products split exp(G_r - G_s) around the first row of a 16-row
  // block, so a factor reaches exp(15 |L|); it must stay finite in fp32
  // (ln FLT_MAX = 88.72), which holds for |L| <= kMaxGateBound.
  if (p->gate_lower_bound < -kMaxGateBound) return KDA_ERR_UNSUPPORTED;
  if (!(p->l2_eps >= 0.f) || !std::isfinite(p->l2_eps) || !std::isfinite(p->scale))
    return KDA_ERR_INVALID;
  if (p->seg_chunks < 0 || p->chunk < 1) return KDA_ERR_INVALID;
  if (p->dtype != KDA_F32 && p->dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  const int gmap = p->gate_mode & ~KDA_GATE_PER_HEAD;
  if (gmap != KDA_GATE_SIGMOID_BOUND && gmap != KDA_GATE_SOFTPLUS_CLAMP)
    return KDA_ERR_UNSUPPORTED;
  if (p->K != p->V) return KDA_ERR_UNSUPPORTED;
  if (!supported(p->dtype, p->K, p->chunk)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

// GDN-2 is built for the per-channel gate, at every size KDA is built for
// except fp32 with K = 64 and 64-token chunks (its gradient kernel's tiles
// exceed the LDS there).
bool gdn2_supported(const kda_problem* p) {
  if (p->gate_mode & KDA_GATE_PER_HEAD) return false;
  return !(p->dtype == KDA_F32 && p->K == 64 && p->chunk == 64);
}

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// One segment of a plan (Seg in kda_internal.h, host side).
struct SegInfo {
  int c0, c1;  // chunk-order indices
  int n0, n1;  // sequences that may have chunks in it
  int active;  // sequences that have
  int pos0;    // plan by windows: position of every sequence's first chunk in it
};

struct Plan {
  int N, H, D, C, dtype;
  int64_t T;
  int NC;      // chunks over all sequences
  int seg;     // segment length: chunks (sequence order), or chunks of each sequence (windows)
  int NS;      // number of segments
  bool win;    // plan by windows
  int segmax;  // most chunks in one segment (the operand buffers hold that many)
  int xslots;  // state slots of each carry buffer
  int nck;     // checkpoint slots
  size_t esz;  // operand element size
  std::vector<SegInfo> segs;
};

size_t fwd_ops_per(const Plan& P) {  // bytes per (chunk, head), forward operands
  const size_t C = P.C, K = P.D;
  return (3 * C * K + C * C * (P.esz == 2 ? 2 : 1)) * P.esz + C * K * 4 + K * 4;
}
size_t bwd_ops_per(const Plan& P) {  // backward operands + recorded states
  const size_t C = P.C, K = P.D;
  return (6 * C * K + 3 * C * C) * P.esz + K * 4 + (2 * K * K + 2 * C * K) * P.esz;
}

size_t budget_bytes() {
  const char* e = std::getenv("KDA_WS_BUDGET_MB");
  long mb = e ? std::atol(e) : 1024;
  if (mb < 1) mb = 1;
  return static_cast<size_t>(mb) << 20;
}

// Largest table of sequence starts per segment a plan by windows may use
// (segments x (sequences + 1) entries).
constexpr int64_t kMaxWindowTable = 1 << 20;

// Segments of at most `cap` chunks. Two plans:
//   sequence order: the chunk order lists the sequences one after another
//     and a segment is a run of `seg` chunks of it, so at most one sequence
//     crosses each boundary;
//   windows: segment sg holds chunks [sg w, (sg + 1) w) of every sequence,
//     so each segment's scans run every sequence at once over w chunks.
// The scans walk each segment's chunks one after another per (sequence,
// head), so a plan's critical path is the sum over its segments of the most
// chunks one sequence has in it: windows are taken when that is at most
// three quarters of the sequence-order plan's (several long sequences in a
// packed batch; a single sequence gives both plans the same segments), and
// when the states they hold fit: every sequence crossing a window boundary
// needs a carry slot and, in the backward, a checkpoint per window start, each
// a [H][K][V] fp32 state. The windows' operands, carries and checkpoints must
// stay within the budget or within what the sequence-order plan holds.
Plan make_plan(const kda_problem* p, bool bwd) {
  Plan P{};
  P.N = p->n_seqs;
  P.H = p->H;
  P.D = p->K;
  P.C = p->chunk;
  P.dtype = p->dtype;
  P.T = p->total_tokens;
  P.esz = p->dtype == KDA_BF16 ? 2 : 4;
  const int N = P.N;
  std::vector<int> nc(N), coff(N + 1, 0);
  int act = 0, maxnc = 0;
  for (int n = 0; n < N; ++n) {
    nc[n] = (p->cu_seqlens_host[n + 1] - p->cu_seqlens_host[n] + P.C - 1) / P.C;
    coff[n + 1] = coff[n] + nc[n];
    act += nc[n] > 0;
    maxnc = nc[n] > maxnc ? nc[n] : maxnc;
  }
  P.NC = coff[N];
  const size_t per = (bwd ? bwd_ops_per(P) : fwd_ops_per(P)) * P.H;
  int cap, seg;
  if (p->seg_chunks > 0) {
    cap = seg = p->seg_chunks;
  } else {
    // the fewest segments that fit the budget, then equal segment lengths
    // (no short last segment: every launch fills the same number of rounds)
    const size_t fit = budget_bytes() / per;
    cap = static_cast<int>(fit < 1 ? 1 : (fit > static_cast<size_t>(P.NC) ? P.NC : fit));
    const int ns = (P.NC + cap - 1) / cap;
    seg = (P.NC + ns - 1) / ns;
  }
  if (seg > P.NC) seg = P.NC;
  if (seg < 1) seg = 1;
  // sequence order
  const int ns_seq = (P.NC + seg - 1) / seg;
  std::vector<SegInfo> sq(ns_seq);
  int64_t cost_seq = 0;
  for (int sg = 0, n = 0; sg < ns_seq; ++sg) {
    SegInfo& e = sq[sg];
    e.c0 = sg * seg;
    e.c1 = e.c0 + seg < P.NC ? e.c0 + seg : P.NC;
    e.pos0 = 0;
    while (coff[n + 1] <= e.c0) ++n;  // first sequence with a chunk at or after c0
    e.n0 = n;
    e.active = 0;
    int m = n, run = 0;
    for (; m < N && coff[m] < e.c1; ++m) {
      const int lo = coff[m] > e.c0 ? coff[m] : e.c0, hi = coff[m + 1] < e.c1 ? coff[m + 1] : e.c1;
      if (hi > lo) {
        ++e.active;
        run = hi - lo > run ? hi - lo : run;
      }
    }
    e.n1 = m;
    cost_seq += run;
  }
  P.win = false;
  if (ns_seq > 1 && act >= 2 && act <= cap) {
    auto held = [&](int w) {  // chunks of a window-w segment 0
      int64_t t = 0;
      for (int n = 0; n < N; ++n) t += nc[n] < w ? nc[n] : w;
      return t;
    };
    int lo = 1, hi = maxnc;  // held(lo) <= cap
    while (lo < hi) {
      const int mid = lo + (hi - lo + 1) / 2;
      if (held(mid) <= cap) lo = mid; else hi = mid - 1;
    }
    const int nsw = (maxnc + lo - 1) / lo, w = (maxnc + nsw - 1) / nsw;
    const size_t slot = up(static_cast<size_t>(P.H) * P.D * P.D * 4);
    int64_t cross = 0, cks = 0;  // sequences longer than a window; their window starts
    for (int n = 0; n < N; ++n) {
      cross += nc[n] > w;
      cks += nc[n] > w ? (nc[n] + w - 1) / w - 1 : 0;
    }
    const size_t mem_w = static_cast<size_t>(held(w)) * per +
                         static_cast<size_t>(2 * cross + (bwd ? cks : 0)) * slot;
    const size_t mem_seq = static_cast<size_t>(seg) * per + (2 + (bwd ? ns_seq : 0)) * slot;
    const size_t mem_cap = budget_bytes() > mem_seq ? budget_bytes() : mem_seq;
    if (static_cast<int64_t>(nsw) * (N + 1) <= kMaxWindowTable && 4LL * maxnc <= 3 * cost_seq &&
        mem_w <= mem_cap) {
      P.win = true;
      P.seg = w;
      P.NS = nsw;
      P.segs.resize(nsw);
      int64_t below = 0;  // chunks at positions below sg * w
      for (int sg = 0; sg < nsw; ++sg) {
        SegInfo& e = P.segs[sg];
        e.pos0 = sg * w;
        e.n0 = N;
        e.n1 = 0;
        e.active = 0;
        int64_t in = 0;
        for (int n = 0; n < N; ++n) {
          const int k = nc[n] - e.pos0;
          if (k <= 0) continue;
          in += k < w ? k : w;
          ++e.active;
          e.n0 = n < e.n0 ? n : e.n0;
          e.n1 = n + 1;
        }
        e.c0 = static_cast<int>(below);
        e.c1 = static_cast<int>(below + in);
        below += in;
      }
      P.segmax = P.segs[0].c1 - P.segs[0].c0;
      P.xslots = 0;
      P.nck = 0;
      for (int n = 0; n < N; ++n) {
        P.xslots += nc[n] > w;
        P.nck += nc[n] > w ? (nc[n] + w - 1) / w - 1 : 0;
      }
      if (P.xslots < 1) P.xslots = 1;
      if (P.nck < 1) P.nck = 1;
    }
  }
  if (!P.win) {
    P.seg = seg;
    P.NS = ns_seq;
    P.segs = std::move(sq);
    P.segmax = seg;
    P.xslots = 1;
    P.nck = ns_seq;
  }
  return P;
}

// Carve a ChunkOps (forward or backward layout) for `seg` chunks from *cur.
ChunkOps carve_ops(const Plan& P, bool bwd, unsigned char*& cur) {
  const size_t n = static_cast<size_t>(P.segmax) * P.H;
  const size_t C = P.C, K = P.D, e = P.esz;
  ChunkOps o{};
  auto take = [&](size_t bytes) { void* r = cur; cur += up(bytes); return r; };
  o.Wn = take(n * C * K * e);
  o.kgT = take(n * K * C * e);
  o.gam = static_cast<float*>(take(n * K * 4));
  if (!bwd) {
    o.Uf = static_cast<float*>(take(n * C * K * 4));
    o.qg = take(n * C * K * e);
    o.Aqk = take(n * C * C * e);
    if (e == 2) o.Aqk_lo = take(n * C * C * e);
  } else {
    o.U = take(n * C * K * e);
    o.AqkT = take(n * C * C * e);
    o.kg = take(n * C * K * e);
    o.qgT = take(n * K * C * e);
    o.WnT = take(n * K * C * e);
    o.TT = take(n * C * C * e);
    o.PT = take(n * C * C * e);
  }
  return o;
}

size_t ops_bytes(const Plan& P, bool bwd) {
  unsigned char* cur = nullptr;
  carve_ops(P, bwd, cur);
  return reinterpret_cast<size_t>(cur);
}

size_t states_bytes(const Plan& P) {
  const size_t n = static_cast<size_t>(P.segmax) * P.H, C = P.C, K = P.D, e = P.esz;
  return up(n * K * K * e) * 2 + up(n * C * K * e) * 2;
}

size_t state_slot(const Plan& P) { return up(static_cast<size_t>(P.H) * P.D * P.D * 4); }

// The chunk table at the workspace start (TableArgs in kda_internal.h):
// coff [N+1], cloc [NC], ckt [N]; for a plan by windows also xr [N] and
// pst [NS][N+1].
size_t table_bytes(const Plan& P) {
  size_t b = up((P.N + 1) * 4) + up(static_cast<size_t>(P.NC > 0 ? P.NC : 1) * 8) +
             up(static_cast<size_t>(P.N) * 8);
  if (P.win) b += up(static_cast<size_t>(P.N) * 4) + up(static_cast<size_t>(P.NS) * (P.N + 1) * 4);
  return b;
}
struct Table {
  int32_t* coff;
  int2* cloc;
  int2* ckt;
  int32_t* xr;
  int32_t* pst;
};
Table carve_table(const Plan& P, unsigned char*& cur) {
  unsigned char* c = cur;
  auto take = [&](size_t bytes) { unsigned char* r = c; c += up(bytes); return r; };
  Table t{};
  t.coff = reinterpret_cast<int32_t*>(take((P.N + 1) * 4));
  t.cloc = reinterpret_cast<int2*>(take(static_cast<size_t>(P.NC > 0 ? P.NC : 1) * 8));
  t.ckt = reinterpret_cast<int2*>(take(static_cast<size_t>(P.N) * 8));
  if (P.win) {
    t.xr = reinterpret_cast<int32_t*>(take(static_cast<size_t>(P.N) * 4));
    t.pst = reinterpret_cast<int32_t*>(take(static_cast<size_t>(P.NS) * (P.N + 1) * 4));
  }
  cur += table_bytes(P);
  return t;
}
// Chunk-table launch arguments: plan P's table, with the checkpoint layout
// of plan CK (the backward's plan).
TableArgs table_args(const Plan& P, const Plan& CK, const Table& t, const int32_t* cu) {
  TableArgs a{};
  a.cu = cu;
  a.N = P.N;
  a.C = P.C;
  a.NC = P.NC;
  a.win = P.win ? P.seg : 0;
  a.NS = P.NS;
  a.ck_every = CK.seg;
  a.ck_win = CK.win ? 1 : 0;
  a.coff = t.coff;
  a.cloc = t.cloc;
  a.ckt = t.ckt;
  a.xr = t.xr;
  a.pst = t.pst;
  return a;
}
Seg seg_of(const Plan& P, const Table& t, int sg) {
  const SegInfo& e = P.segs[sg];
  return Seg{e.c0, e.c1, e.n0, e.n1,
             P.win ? t.pst + static_cast<size_t>(sg) * (P.N + 1) : nullptr, e.pos0};
}

size_t fwd_bytes(const Plan& P) {
  return table_bytes(P) + 2 * P.xslots * state_slot(P) + ops_bytes(P, false);
}

size_t bwd_bytes(const Plan& P) {
  const size_t ops = ops_bytes(P, true) > ops_bytes(P, false) ? ops_bytes(P, true) : ops_bytes(P, false);
  return table_bytes(P) + up(static_cast<size_t>(P.NC) * P.H * (P.D + 1) * 8) +
         static_cast<size_t>(P.nck) * state_slot(P) + 2 * P.xslots * state_slot(P) + ops +
         states_bytes(P);
}

bool has_empty_sequence(const kda_problem* p) {
  for (int n = 0; n < p->n_seqs; ++n)
    if (p->cu_seqlens_host[n + 1] == p->cu_seqlens_host[n]) return true;
  return false;
}

int hip_fail(hipError_t e) {
  std::snprintf(g_msg, sizeof g_msg, "HIP launch failed: %s", hipGetErrorString(e));
  return KDA_ERR_HIP;
}

// Per-kernel timing (kda_profile_begin / kda_profile_end): event pairs
// recorded on the launch stream around each launch of the calling thread.
struct ProfRec {
  int kind;
  int64_t units;
  hipEvent_t a, b;
};
thread_local bool g_prof_on = false;
thread_local std::vector<ProfRec> g_prof;

struct ProfScope {
  int kind;
  int64_t units;
  hipStream_t s;
  hipEvent_t a = nullptr;
  ProfScope(int k, int64_t u, hipStream_t st) : kind(k), units(u), s(st) {
    if (g_prof_on && hipEventCreate(&a) == hipSuccess && hipEventRecord(a, s) != hipSuccess) {
      (void)hipEventDestroy(a);
      a = nullptr;
    }
  }
  void done() {
    if (!a) return;
    hipEvent_t b = nullptr;
    if (hipEventCreate(&b) == hipSuccess && hipEventRecord(b, s) == hipSuccess) {
      g_prof.push_back({kind, units, a, b});
    } else {
      if (b) (void)hipEventDestroy(b);
      (void)hipEventDestroy(a);
    }
    a = nullptr;
  }
};

#define KDA_TRY(kind, units, expr)             \
  do {                                         \
    ProfScope ps_(kind, units, s);             \
    const hipError_t e_ = (expr);              \
    ps_.done();                                \
    if (e_ != hipSuccess) return hip_fail(e_); \
  } while (0)

Dims make_dims(const kda_problem* p) {
  Dims d{};
  d.N = p->n_seqs;
  d.H = p->H;
  d.scale = p->scale;
  d.lb = p->gate_lower_bound;
  d.eps = p->l2_eps;
  d.gate_mode = p->gate_mode & ~KDA_GATE_PER_HEAD;
  d.gate_head = (p->gate_mode & KDA_GATE_PER_HEAD) ? 1 : 0;
  return d;
}

}  // namespace

extern "C" {

int kda_check_problem(const kda_problem* p) { return check_problem(p); }

size_t kda_fwd_workspace_bytes(const kda_problem* p) {
  if (check_problem(p) != KDA_OK) return 0;
  return fwd_bytes(make_plan(p, false));
}

size_t kda_bwd_workspace_bytes(const kda_problem* p) {
  if (check_problem(p) != KDA_OK) return 0;
  return bwd_bytes(make_plan(p, true));
}

size_t kda_prologue_workspace_bytes(const kda_problem* p) {
  if (check_problem(p) != KDA_OK) return 0;
  return table_bytes(make_plan(p, false));
}

int kda_prologue(const kda_problem* p, const void* q, const void* k, const void* raw_g,
                 const void* raw_beta, const float* A_log, const float* dt_bias,
                 const int32_t* cu_seqlens, float* qh, float* kh, float* beta, float* gcum,
                 void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_problem(p);
  if (st != KDA_OK) return st;
  if (!q || !k || !raw_g || !raw_beta || !A_log || !dt_bias || !cu_seqlens || !qh || !kh ||
      !beta || !gcum || !workspace)
    return KDA_ERR_INVALID;
  if (workspace_bytes < kda_prologue_workspace_bytes(p)) return KDA_ERR_WORKSPACE;
  const Plan P = make_plan(p, false);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* cur = static_cast<unsigned char*>(workspace);
  const Table tb = carve_table(P, cur);
  Inputs in{q, k, nullptr, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, tb.coff, tb.cloc};
  KDA_TRY(KDA_KERNEL_CHUNK_TABLE, 0, launch_chunk_table(table_args(P, P, tb, cu_seqlens), s));
  if (P.NC > 0)
    KDA_TRY(KDA_KERNEL_PROLOGUE, static_cast<int64_t>(P.NC) * P.H, launch_prologue(P.dtype, P.D, P.C, make_dims(p), in, P.NC, qh, kh, beta, gcum, s));
  return KDA_OK;
}

int32_t kda_bwd_segment_chunks(const kda_problem* p) {
  if (check_problem(p) != KDA_OK) return 0;
  return make_plan(p, true).seg;
}

size_t kda_checkpoint_bytes(const kda_problem* p) {
  if (check_problem(p) != KDA_OK) return 0;
  const Plan P = make_plan(p, true);
  return static_cast<size_t>(P.nck) * state_slot(P);
}

}  // extern "C"

namespace {

// The forward of KDA (raw_beta) or of GDN-2 (g2: raw_b, raw_w).
int fwd_common(bool g2, const kda_problem* p, const void* q, const void* k, const void* v,
               const void* raw_g, const void* raw_beta, const void* raw_b, const void* raw_w,
               const float* A_log, const float* dt_bias, const int32_t* cu_seqlens, void* o,
               const kda_state_io* io, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_problem(p);
  if (st != KDA_OK) return st;
  if (!q || !k || !v || !raw_g || !A_log || !dt_bias || !cu_seqlens || !o || !workspace)
    return KDA_ERR_INVALID;
  if (g2 ? (!raw_b || !raw_w) : !raw_beta) return KDA_ERR_INVALID;
  if (g2 && !gdn2_supported(p)) return KDA_ERR_UNSUPPORTED;
  const Plan P = make_plan(p, false);
  if (workspace_bytes < fwd_bytes(P)) return KDA_ERR_WORKSPACE;
  const kda_state_io none{};
  if (!io) io = &none;
  const Plan PB = make_plan(p, true);  // the backward's segments (checkpoints)
  if (io->ckpt && io->ckpt_bytes < kda_checkpoint_bytes(p)) return KDA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* cur = static_cast<unsigned char*>(workspace);
  const Table tb = carve_table(P, cur);
  // a single backward segment needs no checkpoint
  const ScanStates ss{io->h0, io->ht, PB.NS > 1 ? io->ckpt : nullptr,
                      CarryMap{tb.ckt, PB.seg, nullptr, PB.nck}};
  float* carry[2];
  carry[0] = reinterpret_cast<float*>(cur);
  cur += P.xslots * state_slot(P);
  carry[1] = reinterpret_cast<float*>(cur);
  cur += P.xslots * state_slot(P);
  const CarryMap cm{nullptr, 0, tb.xr, P.xslots};
  const ChunkOps ops = carve_ops(P, false, cur);
  Dims d = make_dims(p);
  d.gdn2 = g2 ? 1 : 0;
  Inputs in{q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, tb.coff, tb.cloc};
  in.bk = raw_b;
  in.wv = raw_w;
  KDA_TRY(KDA_KERNEL_CHUNK_TABLE, 0, launch_chunk_table(table_args(P, PB, tb, cu_seqlens), s));
  for (int sg = 0; sg < P.NS; ++sg) {
    const Seg sd = seg_of(P, tb, sg);
    const int64_t units = static_cast<int64_t>(sd.c1 - sd.c0) * P.H;
    const int act = P.segs[sg].active;
    KDA_TRY(KDA_KERNEL_CHUNK_LOCAL, units, launch_chunk_local(P.dtype, P.D, P.C, KL_FWD, d, in, sd.c0, sd.c1 - sd.c0, ops, s));
    KDA_TRY(KDA_KERNEL_SCAN_FWD, units, launch_scan_fwd(P.dtype, P.D, P.C, d, in, sd, act, ops, o, nullptr, carry[sg & 1],
                            carry[(sg + 1) & 1], cm, ss, s));
  }
  if (io->ht && has_empty_sequence(p))
    KDA_TRY(KDA_KERNEL_CHUNK_TABLE, 0, launch_state_passthrough(cu_seqlens, P.N, P.H, P.D * P.D, io->h0, io->ht, s));
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_fwd_ex(const kda_problem* p, const void* q, const void* k, const void* v,
               const void* raw_g, const void* raw_beta, const float* A_log,
               const float* dt_bias, const int32_t* cu_seqlens, void* o,
               const kda_state_io* io, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_common(false, p, q, k, v, raw_g, raw_beta, nullptr, nullptr, A_log, dt_bias, cu_seqlens,
                    o, io, workspace, workspace_bytes, stream);
}

int kda_gdn2_fwd(const kda_problem* p, const void* q, const void* k, const void* v,
                 const void* raw_g, const void* raw_b, const void* raw_w, const float* A_log,
                 const float* dt_bias, const int32_t* cu_seqlens, void* o, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return fwd_common(true, p, q, k, v, raw_g, nullptr, raw_b, raw_w, A_log, dt_bias, cu_seqlens, o,
                    nullptr, workspace, workspace_bytes, stream);
}

int kda_fwd(const kda_problem* p, const void* q, const void* k, const void* v,
            const void* raw_g, const void* raw_beta, const float* A_log, const float* dt_bias,
            const int32_t* cu_seqlens, void* o, void* workspace, size_t workspace_bytes,
            void* stream) {
  return kda_fwd_ex(p, q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, o, nullptr,
                    workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The backward of KDA (raw_beta, draw_beta) or of GDN-2 (g2: raw_b, raw_w,
// draw_b in draw_beta's place, draw_w).
int bwd_common(bool g2, const kda_problem* p, const void* q, const void* k, const void* v,
               const void* raw_g, const void* raw_beta, const void* raw_b, const void* raw_w,
               const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
               const void* dO, void* dq, void* dk, void* dv, void* draw_g, void* draw_beta,
               void* draw_w, float* dA_log, float* ddt_bias, const kda_state_io* io,
               void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_problem(p);
  if (st != KDA_OK) return st;
  if (!q || !k || !v || !raw_g || !A_log || !dt_bias || !cu_seqlens || !dO || !dq || !dk ||
      !dv || !draw_g || !draw_beta || !dA_log || !ddt_bias || !workspace)
    return KDA_ERR_INVALID;
  if (g2 ? (!raw_b || !raw_w || !draw_w) : !raw_beta) return KDA_ERR_INVALID;
  if (g2 && !gdn2_supported(p)) return KDA_ERR_UNSUPPORTED;
  const Plan P = make_plan(p, true);
  if (workspace_bytes < bwd_bytes(P)) return KDA_ERR_WORKSPACE;
  const kda_state_io none{};
  if (!io) io = &none;
  if (io->ckpt && io->ckpt_bytes < kda_checkpoint_bytes(p)) return KDA_ERR_WORKSPACE;
  const ScanStates fwd_ss{io->h0, nullptr, nullptr, CarryMap{}};
  const ScanStates bwd_ss{io->dht, io->dh0, nullptr, CarryMap{}};
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* cur = static_cast<unsigned char*>(workspace);
  const Table tb = carve_table(P, cur);
  double* partials = reinterpret_cast<double*>(cur);
  cur += up(static_cast<size_t>(P.NC) * P.H * (P.D + 1) * 8);
  // states entering the segments (checkpoint layout of ckt); the forward's
  // checkpoints when given
  float* ckpt = io->ckpt ? io->ckpt : reinterpret_cast<float*>(cur);
  cur += static_cast<size_t>(P.nck) * state_slot(P);
  const CarryMap ck_map{tb.ckt, P.seg, nullptr, P.nck};
  float* dcarry[2];
  dcarry[0] = reinterpret_cast<float*>(cur);
  cur += P.xslots * state_slot(P);
  dcarry[1] = reinterpret_cast<float*>(cur);
  cur += P.xslots * state_slot(P);
  const CarryMap cm{nullptr, 0, tb.xr, P.xslots};
  unsigned char* ops_base = cur;
  unsigned char* c2 = ops_base;
  const ChunkOps ops_b = carve_ops(P, true, c2);
  unsigned char* c3 = ops_base;
  const ChunkOps ops_f = carve_ops(P, false, c3);  // overlays ops_b (checkpoint pass only)
  cur = ops_base + (ops_bytes(P, true) > ops_bytes(P, false) ? ops_bytes(P, true) : ops_bytes(P, false));
  SegStates sts{};
  {
    const size_t n = static_cast<size_t>(P.segmax) * P.H, C = P.C, K = P.D, e = P.esz;
    sts.h = cur;
    cur += up(n * K * K * e);
    sts.dh = cur;
    cur += up(n * K * K * e);
    sts.Vn = cur;
    cur += up(n * C * K * e);
    sts.dVnT = cur;
    cur += up(n * C * K * e);
  }
  Dims d = make_dims(p);
  d.gdn2 = g2 ? 1 : 0;
  Inputs in{q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, tb.coff, tb.cloc};
  in.bk = raw_b;
  in.wv = raw_w;
  KDA_TRY(KDA_KERNEL_CHUNK_TABLE, 0, launch_chunk_table(table_args(P, P, tb, cu_seqlens), s));
  // checkpoint pass: the state entering each segment (skipped when the
  // forward saved them)
  for (int sg = 0; !io->ckpt && sg + 1 < P.NS; ++sg) {
    const Seg sd = seg_of(P, tb, sg);
    const int64_t units = static_cast<int64_t>(sd.c1 - sd.c0) * P.H;
    KDA_TRY(KDA_KERNEL_CHUNK_LOCAL_STATE, units, launch_chunk_local(P.dtype, P.D, P.C, KL_STATE, d, in, sd.c0, sd.c1 - sd.c0, ops_f, s));
    KDA_TRY(KDA_KERNEL_SCAN_STATE, units, launch_scan_fwd(P.dtype, P.D, P.C, d, in, sd, P.segs[sg].active, ops_f, nullptr, nullptr,
                            ckpt, ckpt, ck_map, fwd_ss, s));
  }
  for (int sg = P.NS - 1; sg >= 0; --sg) {
    const Seg sd = seg_of(P, tb, sg);
    const int64_t units = static_cast<int64_t>(sd.c1 - sd.c0) * P.H;
    const int act = P.segs[sg].active;
    KDA_TRY(KDA_KERNEL_CHUNK_LOCAL_BWD, units, launch_chunk_local(P.dtype, P.D, P.C, KL_BWD, d, in, sd.c0, sd.c1 - sd.c0, ops_b, s));
    // the recording scan writes no carry: the next segment's entering state is known
    KDA_TRY(KDA_KERNEL_SCAN_REC, units, launch_scan_fwd(P.dtype, P.D, P.C, d, in, sd, act, ops_b, nullptr, &sts,
                            ckpt, nullptr, ck_map, fwd_ss, s));
    KDA_TRY(KDA_KERNEL_SCAN_BWD, units, launch_scan_bwd(P.dtype, P.D, P.C, d, in, dO, sd, act, ops_b, sts,
                            dcarry[(sg + 1) & 1], dcarry[sg & 1], cm, bwd_ss, s));
    KDA_TRY(KDA_KERNEL_CHUNK_GRAD, units, launch_chunk_grad(P.dtype, P.D, P.C, d, in, dO, sd.c0, sd.c1 - sd.c0, ops_b, sts, dq, dk, dv,
                              draw_g, draw_beta, draw_w, partials, s));
  }
  KDA_TRY(KDA_KERNEL_GATE_REDUCE, 0, launch_gate_reduce(P.D, P.H, P.NC, d.gate_head, partials, dA_log, ddt_bias, s));
  if (io->dh0 && has_empty_sequence(p))
    KDA_TRY(KDA_KERNEL_CHUNK_TABLE, 0, launch_state_passthrough(cu_seqlens, P.N, P.H, P.D * P.D, io->dht, io->dh0, s));
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_bwd_ex(const kda_problem* p, const void* q, const void* k, const void* v,
               const void* raw_g, const void* raw_beta, const float* A_log,
               const float* dt_bias, const int32_t* cu_seqlens, const void* dO, void* dq,
               void* dk, void* dv, void* draw_g, void* draw_beta, float* dA_log,
               float* ddt_bias, const kda_state_io* io, void* workspace,
               size_t workspace_bytes, void* stream) {
  return bwd_common(false, p, q, k, v, raw_g, raw_beta, nullptr, nullptr, A_log, dt_bias, cu_seqlens,
                    dO, dq, dk, dv, draw_g, draw_beta, nullptr, dA_log, ddt_bias, io, workspace,
                    workspace_bytes, stream);
}

int kda_gdn2_bwd(const kda_problem* p, const void* q, const void* k, const void* v,
                 const void* raw_g, const void* raw_b, const void* raw_w, const float* A_log,
                 const float* dt_bias, const int32_t* cu_seqlens, const void* dO, void* dq,
                 void* dk, void* dv, void* draw_g, void* draw_b, void* draw_w, float* dA_log,
                 float* ddt_bias, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(true, p, q, k, v, raw_g, nullptr, raw_b, raw_w, A_log, dt_bias, cu_seqlens, dO,
                    dq, dk, dv, draw_g, draw_b, draw_w, dA_log, ddt_bias, nullptr, workspace,
                    workspace_bytes, stream);
}

int kda_bwd(const kda_problem* p, const void* q, const void* k, const void* v,
            const void* raw_g, const void* raw_beta, const float* A_log, const float* dt_bias,
            const int32_t* cu_seqlens, const void* dO, void* dq, void* dk, void* dv,
            void* draw_g, void* draw_beta, float* dA_log, float* ddt_bias, void* workspace,
            size_t workspace_bytes, void* stream) {
  return kda_bwd_ex(p, q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, dO, dq, dk, dv,
                    draw_g, draw_beta, dA_log, ddt_bias, nullptr, workspace, workspace_bytes,
                    stream);
}

int kda_profile_begin(void) {
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  g_prof_on = true;
  return KDA_OK;
}

int kda_profile_end(int32_t* launches, double* total_ms, int64_t* units, int n) {
  g_prof_on = false;
  for (int k = 0; k < n; ++k) {
    if (launches) launches[k] = 0;
    if (total_ms) total_ms[k] = 0.0;
    if (units) units[k] = 0;
  }
  int st = KDA_OK;
  for (auto& r : g_prof) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      st = KDA_ERR_HIP;
    if (r.kind >= 0 && r.kind < n) {
      if (launches) launches[r.kind] += 1;
      if (total_ms) total_ms[r.kind] += ms;
      if (units) units[r.kind] += r.units;
    }
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  return st;
}

const char* kda_kernel_name(int kind) {
  static const char* names[KDA_KERNEL_COUNT] = {
      "chunk_table", "prologue",        "chunk_local",       "scan_fwd",
      "scan_bwd",    "chunk_grad",      "gate_reduce",       "chunk_local_bwd",
      "chunk_local_state", "scan_rec",  "scan_state"};
  return (kind >= 0 && kind < KDA_KERNEL_COUNT) ? names[kind] : "unknown";
}

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported K/V/chunk/dtype/gate combination";
    case KDA_ERR_WORKSPACE: return "workspace too small";
    case KDA_ERR_HIP: return g_msg[0] ? g_msg : "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
