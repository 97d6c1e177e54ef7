// C-ABI host library of the Key-Value Means attention layer (see include/kvm.h).
//
// Host responsibilities: argument checks (before anything is queued), the
// data-independent size schedule, carving the caller's workspace, and queueing
// the gfx950 kernels on the caller's stream.  No device allocation, no host
// synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <climits>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kvm.h"
#include "kvm_internal.h"

enum Phase { kScan = 0, kAttn, kRing, kDecAbsorb, kDecAttn, kPrep, kPhases };
static_assert(KVM_PROFILE_SCAN == 1 << kScan && KVM_PROFILE_ATTN == 1 << kAttn && KVM_PROFILE_RING == 1 << kRing &&
                  KVM_PROFILE_DEC_ABSORB == 1 << kDecAbsorb && KVM_PROFILE_DEC_ATTN == 1 << kDecAttn &&
                  KVM_PROFILE_PREP == 1 << kPrep && KVM_PROFILE_ALL == (1 << kPhases) - 1,
              "profile masks follow the phase order");

struct kvm_state {
  kvm_config cfg;
  kvm::Dims m;
  kvm::Dev d;
  std::vector<int32_t> sched;      // 4 ints per absorbable chunk: sinks, appends, rows_before, idx_off
  int64_t pos = 0;
  int64_t absorbed = 0;
  // per-sequence positions and absorbed chunks; pos/absorbed above hold while
  // every sequence is at the same position (per_seq false)
  std::vector<int64_t> spos, sabs;
  bool per_seq = false;
  std::vector<int64_t> seqtab;     // host copy of the per-sequence launch table
  bool poisoned = false;
  // profiling: event pairs recorded around kernel phases
  int profiling = 0;     // mask of phases (bit = 1 << Phase) that record events
  struct Rec {
    int phase;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  // prefill overlap: attention of ready query chunks runs on `side` while the
  // scan continues on the caller's stream (fork/join through `sync_ev`)
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> sync_ev;
  ~kvm_state() {
    for (Rec& r : recs) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
    for (hipEvent_t e : sync_ev) (void)hipEventDestroy(e);
    if (side) (void)hipStreamDestroy(side);
  }
};

namespace {

thread_local std::string g_err;

kvm_status fail(kvm_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// Smallest integer r with r*r >= x.
uint64_t ceil_sqrt_u64(uint64_t x) {
  uint64_t r = (uint64_t)std::sqrt((long double)x);
  while (r > 0 && r * r > x) --r;
  while ((r + 1) * (r + 1) <= x) ++r;
  return r * r == x ? r : r + 1;
}

// Rows the schedule wants (sinks included) once T tokens have been absorbed.
int64_t capacity(const kvm_config& c, int64_t T) {
  if (c.sched == KVM_SCHED_FIXED) return c.max_slots;
  if (c.sched == KVM_SCHED_POWER) return (int64_t)std::ceil((double)c.alpha * std::pow((double)T, c.exponent));
  const uint64_t a = (uint64_t)c.alpha;
  const int64_t s = (int64_t)ceil_sqrt_u64(a * a * (uint64_t)T);
  if (c.sched == KVM_SCHED_SQRT) return s;
  return s < c.max_slots ? s : c.max_slots;
}

int64_t max_absorbable_chunks(const kvm_config& c) {
  const int64_t n_chunks = (c.max_tokens + c.chunk - 1) / c.chunk;
  const int64_t j = n_chunks - c.window / c.chunk - 1;
  return j > 0 ? j : 0;
}

// Per absorbed chunk j < n: f(j, sinks created, rows appended, rows before).
template <typename F>
void for_each_chunk(const kvm_config& c, int64_t n, F f) {
  int64_t rows = 0, nsink = 0;
  for (int64_t j = 0; j < n; ++j) {
    const int64_t before = rows;
    int64_t cand = c.chunk;
    const int64_t sk = std::min<int64_t>(c.n_sinks - nsink, cand);
    nsink += sk;
    rows += sk;
    cand -= sk;
    int64_t m = capacity(c, (j + 1) * (int64_t)c.chunk) - rows;
    if (m < 0) m = 0;
    if (m > cand) m = cand;
    rows += m;
    f(j, (int32_t)sk, (int32_t)m, (int32_t)before);
  }
}

void build_schedule(const kvm_config& c, int64_t n, std::vector<int32_t>& sinks, std::vector<int32_t>& app,
                    std::vector<int32_t>& before) {
  sinks.resize(n);
  app.resize(n);
  before.resize(n);
  for_each_chunk(c, n, [&](int64_t j, int32_t sk, int32_t m, int32_t b) {
    sinks[j] = sk;
    app[j] = m;
    before[j] = b;
  });
}

kvm_status validate(const kvm_config* c) {
  if (!c) return fail(KVM_E_INVALID_ARG, "config is NULL");
  if (c->batch < 1 || c->heads < 1) return fail(KVM_E_INVALID_ARG, "batch and heads must be >= 1");
  if ((int64_t)c->batch * c->heads > (1 << 20)) return fail(KVM_E_INVALID_ARG, "batch*heads exceeds 2^20");
  if (c->head_dim != 64) return fail(KVM_E_INVALID_ARG, "head_dim must be 64");
  if (c->rope_dims != 32) return fail(KVM_E_INVALID_ARG, "rope_dims must be 32");
  if (c->chunk != 32 && c->chunk != 64 && c->chunk != 128 && c->chunk != 256)
    return fail(KVM_E_INVALID_ARG, "chunk must be 32, 64, 128 or 256");
  if (c->window <= 0 || c->window % c->chunk != 0) return fail(KVM_E_INVALID_ARG, "window must be a positive multiple of chunk");
  if (c->window > (1 << 20)) return fail(KVM_E_INVALID_ARG, "window exceeds 2^20");
  if (c->n_sinks < 0 || c->n_sinks > c->chunk) return fail(KVM_E_INVALID_ARG, "n_sinks must be in [0, chunk]");
  if (c->sched == KVM_SCHED_FIXED) {
    if (c->max_slots < 1) return fail(KVM_E_INVALID_ARG, "fixed schedule needs max_slots >= 1");
  } else if (c->sched == KVM_SCHED_POWER) {
    if (c->alpha < 1 || c->alpha > 4096) return fail(KVM_E_INVALID_ARG, "alpha must be in [1, 4096]");
    if (!(c->exponent > 0.0 && c->exponent <= 1.0)) return fail(KVM_E_INVALID_ARG, "exponent must be in (0, 1]");
  } else if (c->sched == KVM_SCHED_SQRT || c->sched == KVM_SCHED_SATURATING) {
    if (c->alpha < 1 || c->alpha > 4096) return fail(KVM_E_INVALID_ARG, "alpha must be in [1, 4096]");
    if (c->sched == KVM_SCHED_SATURATING && c->max_slots < 1)
      return fail(KVM_E_INVALID_ARG, "saturating schedule needs max_slots >= 1");
  } else {
    return fail(KVM_E_INVALID_ARG, "unknown schedule");
  }
  if (c->max_tokens < 1 || c->max_tokens > ((int64_t)1 << 31) - 1)
    return fail(KVM_E_INVALID_ARG, "max_tokens must be in [1, 2^31)");
  if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta)) return fail(KVM_E_INVALID_ARG, "rope_theta must be > 0");
  if (!(c->ln_eps >= 0.f) || !std::isfinite(c->ln_eps)) return fail(KVM_E_INVALID_ARG, "ln_eps must be >= 0");
  if (!(c->softmax_scale >= 0.f) || !std::isfinite(c->softmax_scale))
    return fail(KVM_E_INVALID_ARG, "softmax_scale must be >= 0");
  if (c->dtype != KVM_F32 && c->dtype != KVM_BF16) return fail(KVM_E_INVALID_ARG, "dtype must be KVM_F32 or KVM_BF16");
  const uint32_t known = KVM_FLAG_TRACE | KVM_FLAG_NO_VALUE_NORM | KVM_FLAG_NO_SINK_PROTECT | KVM_FLAG_NO_MERGE_GATE |
                         KVM_FLAG_SERIAL_PREFILL;
  if (c->flags & ~known) return fail(KVM_E_INVALID_ARG, "unknown flag bits");
  // Every merged token needs a candidate row: the first chunk with non-sink
  // tokens must be allowed to append at least one row (unprotected sinks are
  // candidates themselves).
  const int64_t J = max_absorbable_chunks(*c);
  const int64_t jfirst = c->n_sinks == c->chunk ? 1 : 0;
  const bool sinks_take_merges = (c->flags & KVM_FLAG_NO_SINK_PROTECT) && c->n_sinks > 0;
  if (!sinks_take_merges && J > jfirst && capacity(*c, (jfirst + 1) * (int64_t)c->chunk) <= c->n_sinks)
    return fail(KVM_E_INVALID_ARG, "schedule leaves no non-sink row for the first merged tokens (capacity <= n_sinks)");
  return KVM_OK;
}

struct Plan {
  kvm::Dims m{};
  std::vector<int32_t> sched;  // 4 per chunk
  // byte offsets
  size_t key_sum, val_sum, count, rho, unit, kread, vread, pkey, pval, prho, pcount, pnorm, idx, krot, tslot, tkind, ring_k,
      ring_v, ring_l, rope_cos, rope_sin, sch, nver, xbuf, xerr, seq, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Sizes and workspace offsets for cfg.  keep_sched: also fill p.sched (host memory);
// without it nothing is allocated.
kvm_status plan(const kvm_config* c, Plan& p, bool keep_sched = true) {
  kvm_status st = validate(c);
  if (st != KVM_OK) return st;
  const int64_t J = max_absorbable_chunks(*c);
  int64_t S_cap = 0, idx_total = 0;
  bool too_many = false;
  if (keep_sched) p.sched.assign((size_t)J * 4, 0);
  for_each_chunk(*c, J, [&](int64_t j, int32_t sk, int32_t app, int32_t before) {
    const int64_t after = (int64_t)before + sk + app;
    if (keep_sched) {
      p.sched[4 * j + 0] = sk;
      p.sched[4 * j + 1] = app;
      p.sched[4 * j + 2] = before;
      p.sched[4 * j + 3] = (int32_t)idx_total;
    }
    idx_total += after;
    if (after > S_cap) S_cap = after;
    if (idx_total >= ((int64_t)1 << 31)) too_many = true;
  });
  if (too_many) return fail(KVM_E_INVALID_ARG, "index lists exceed 2^31 entries; lower max_tokens");
  if (S_cap > (1 << 22)) return fail(KVM_E_INVALID_ARG, "state would exceed 2^22 rows");
  kvm::Dims& m = p.m;
  m.BH = c->batch * c->heads;
  m.C = c->chunk;
  m.W = c->window;
  m.R = c->window + c->chunk;
  m.ns = c->n_sinks;
  m.S_cap = (int)S_cap;
  m.J_cap = (int)J;
  m.V_cap = J * c->chunk;
  m.idx_total = idx_total;
  m.max_tokens = c->max_tokens;
  m.scale = c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / std::sqrt((float)c->head_dim);
  m.ln_eps = c->ln_eps;
  m.bf16 = c->dtype == KVM_BF16;
  m.trace = (c->flags & KVM_FLAG_TRACE) ? 1 : 0;
  m.no_vnorm = (c->flags & KVM_FLAG_NO_VALUE_NORM) ? 1 : 0;
  m.unprot = (c->flags & KVM_FLAG_NO_SINK_PROTECT) ? 1 : 0;
  m.no_gate = (c->flags & KVM_FLAG_NO_MERGE_GATE) ? 1 : 0;
  // Scan workgroups per sequence: enough for about 128 workgroups in all (the
  // rest of the chip runs the attention beside the scan), at most 8, and only
  // if each workgroup's share of the rows (every P-th 32-row tile) fits its
  // LDS cache of unit directions; else one workgroup per sequence.
  {
    int want = 0;
    while (want < 3 && (int64_t)m.BH << (want + 1) <= 128) ++want;
    const int64_t lb = m.unprot ? 0 : m.ns;
    const int64_t ntile = S_cap > lb ? (S_cap - lb + 31) / 32 : 0;
    const int64_t own_rows = ((ntile + (1 << want) - 1) >> want) * 32;
    m.Psh = want > 0 && own_rows <= kvm::scan_lds_rows(m.C, m.bf16) ? want : 0;
    m.P = 1 << m.Psh;
  }
  const size_t es = m.bf16 ? 2 : 4;
  const size_t BH = (size_t)m.BH, S = (size_t)S_cap;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  p.key_sum = take(BH * S * 32 * 4);
  p.val_sum = take(BH * S * 64 * 4);
  p.count = take(BH * S * 4);
  p.rho = take(BH * S * 4);
  p.unit = take(BH * S * 128);
  p.kread = take(BH * S * 32 * es);
  p.vread = take(BH * S * 64 * es);
  p.pkey = take(BH * (size_t)m.V_cap * 32 * es);
  p.pval = take(BH * (size_t)m.V_cap * 64 * es);
  p.prho = take(BH * (size_t)m.V_cap * 4);
  p.pcount = take(BH * (size_t)m.V_cap * 4);
  p.pnorm = take(BH * (size_t)m.V_cap * 8);
  p.idx = take(BH * (size_t)idx_total * 4);
  p.tslot = take(m.trace ? BH * (size_t)c->max_tokens * 4 : 0);
  p.tkind = take(m.trace ? BH * (size_t)c->max_tokens : 0);
  p.ring_k = take(BH * (size_t)m.R * 64 * es);
  p.ring_v = take(BH * (size_t)m.R * 64 * es);
  p.ring_l = take(BH * (size_t)m.R * 4);
  p.krot = take(m.bf16 && m.C >= 128 ? BH * (size_t)c->max_tokens * 32 * 2 : 0);
  p.rope_cos = take((size_t)c->max_tokens * 16 * 4);
  p.rope_sin = take((size_t)c->max_tokens * 16 * 4);
  p.sch = take((size_t)J * 16);
  p.nver = take(BH * 4);
  p.xbuf = take(BH * 2 * (size_t)m.P * m.C * 8);
  p.xerr = take(4);
  p.seq = take(BH * kvm::kSeqFields * 8);
  p.total = off;
  return KVM_OK;
}

// Device regions of a workspace at `b` laid out by plan `p`.
void carve(const Plan& p, char* b, kvm::Dev& d) {
  d.key_sum = reinterpret_cast<float*>(b + p.key_sum);
  d.val_sum = reinterpret_cast<float*>(b + p.val_sum);
  d.count = reinterpret_cast<int*>(b + p.count);
  d.rho = reinterpret_cast<float*>(b + p.rho);
  d.unit = b + p.unit;
  d.kread = b + p.kread;
  d.vread = b + p.vread;
  d.pkey = b + p.pkey;
  d.pval = b + p.pval;
  d.prho = reinterpret_cast<float*>(b + p.prho);
  d.pcount = reinterpret_cast<int*>(b + p.pcount);
  d.pnorm = reinterpret_cast<float2*>(b + p.pnorm);
  d.idx = reinterpret_cast<int*>(b + p.idx);
  d.tslot = reinterpret_cast<int*>(b + p.tslot);
  d.tkind = reinterpret_cast<uint8_t*>(b + p.tkind);
  d.ring_k = b + p.ring_k;
  d.ring_v = b + p.ring_v;
  d.ring_l = reinterpret_cast<float*>(b + p.ring_l);
  d.rope_cos = reinterpret_cast<float*>(b + p.rope_cos);
  d.krot = p.m.bf16 && p.m.C >= 128 ? b + p.krot : nullptr;
  d.rope_sin = reinterpret_cast<float*>(b + p.rope_sin);
  d.sched = reinterpret_cast<int4*>(b + p.sch);
  d.nver = reinterpret_cast<int*>(b + p.nver);
  d.xbuf = reinterpret_cast<uint2*>(b + p.xbuf);
  d.xerr = reinterpret_cast<int*>(b + p.xerr);
  d.seq = reinterpret_cast<int64_t*>(b + p.seq);
}

kvm_status hip_fail(kvm_state* st, hipError_t e, const char* what) {
  if (st) st->poisoned = true;
  return fail(KVM_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

hipEvent_t take_event(kvm_state* st) {
  if (!st->pool.empty()) {
    hipEvent_t e = st->pool.back();
    st->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` on stream hs, bracketed by an event pair when profiling.
template <typename F>
hipError_t timed(kvm_state* st, int phase, hipStream_t hs, F launch) {
  if (!(st->profiling & (1 << phase))) return launch();
  hipEvent_t a = take_event(st), b = take_event(st);
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, hs);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, hs);
  st->recs.push_back({phase, a, b});
  return e;
}

// The i-th fork/join event of a prefill call (created on first use, reused by later calls:
// a wait binds to the record that precedes it in host order).
hipEvent_t sync_event(kvm_state* st, size_t i) {
  while (st->sync_ev.size() <= i) {
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
    st->sync_ev.push_back(e);
  }
  return st->sync_ev[i];
}

// Absorption [a0, a1) in pieces, each half of what remains (at least
// kMinPiece chunks; a remainder below that joins the last piece): attention
// of the chunks a piece makes ready overlaps the next piece, and only the
// last piece's dependants run after the scan.  Each piece costs a launch and
// a reload of the workgroups' LDS state (~9 us measured on the 350M-shaped
// prefill), so few pieces pay: halving measured 2.34 ms per prefill there
// against 2.44 ms with pieces shrinking by a third.
constexpr int64_t kMinPiece = 8;
std::vector<int64_t> scan_pieces(int64_t a0, int64_t a1) {
  std::vector<int64_t> b{a0};
  while (b.back() < a1) {
    const int64_t rem = a1 - b.back();
    int64_t nb = std::min(a1, b.back() + std::max<int64_t>(kMinPiece, (rem + 1) / 2));
    if (a1 - nb < kMinPiece) nb = a1;
    b.push_back(nb);
  }
  return b;
}

int rows_after(const kvm_state* st, int64_t j) {
  if (j < 0) return 0;
  const int32_t* s = &st->sched[(size_t)j * 4];
  return s[0] + s[1] + s[2];
}

// Chunks absorbed once `pos` tokens have been consumed (by prefill calls or
// decode steps alike): query chunk ceil(pos/C) - 1 has needed every chunk up
// to its own index - W/C - 1.
int64_t absorbed_at(const kvm::Dims& m, int64_t pos) {
  const int64_t a = (pos + m.C - 1) / m.C - m.W / m.C - 1;
  return a > 0 ? a : 0;
}

// Every sequence at the state's one position (after a call that moves them together).
void set_uniform(kvm_state* st) {
  st->spos.assign((size_t)st->m.BH, st->pos);
  st->sabs.assign((size_t)st->m.BH, st->absorbed);
  st->per_seq = false;
}

// After a per-sequence call: back to the one-position form when every sequence agrees.
void sync_uniform(kvm_state* st) {
  const bool same = std::all_of(st->spos.begin(), st->spos.end(), [&](int64_t x) { return x == st->spos[0]; });
  st->per_seq = !same;
  if (same) {
    st->pos = st->spos[0];
    st->absorbed = st->sabs[0];
  }
}

// Upload the per-sequence launch table (small: kSeqFields int64 per sequence).
hipError_t upload_seq(kvm_state* st, hipStream_t hs) {
  return hipMemcpyAsync(st->d.seq, st->seqtab.data(), st->seqtab.size() * 8, hipMemcpyHostToDevice, hs);
}

// Queue the clearing of the counters and exchange buffers the kernels rely on
// (state creation, reset, load).
hipError_t clear_counters(kvm_state* st, bool trace_too, hipStream_t hs) {
  hipError_t e = hipMemsetAsync(st->d.nver, 0, (size_t)st->m.BH * 4, hs);
  if (e == hipSuccess) e = hipMemsetAsync(st->d.xerr, 0, 4, hs);
  if (e == hipSuccess) e = hipMemsetAsync(st->d.xbuf, 0, (size_t)st->m.BH * 2 * st->m.P * st->m.C * 8, hs);
  if (e == hipSuccess && st->m.trace && trace_too) {
    e = hipMemsetAsync(st->d.tslot, 0xFF, (size_t)st->m.BH * st->m.max_tokens * 4, hs);
    if (e == hipSuccess) e = hipMemsetAsync(st->d.tkind, 0xFF, (size_t)st->m.BH * st->m.max_tokens, hs);
  }
  return e;
}

}  // namespace

extern "C" {

kvm_status kvm_workspace_bytes(const kvm_config* cfg, size_t* bytes) {
  try {
    if (!bytes) return fail(KVM_E_INVALID_ARG, "bytes is NULL");
    Plan p;
    kvm_status s = plan(cfg, p);
    if (s != KVM_OK) return s;
    *bytes = p.total;
    return KVM_OK;
  } catch (...) {
    return fail(KVM_E_INVALID_ARG, "host allocation failed");
  }
}

kvm_status kvm_schedule(const kvm_config* cfg, int64_t n_chunks, int32_t* sinks, int32_t* appends, int32_t* rows) {
  try {
    kvm_status s = validate(cfg);
    if (s != KVM_OK) return s;
    if (n_chunks < 0 || n_chunks > (1 << 26)) return fail(KVM_E_INVALID_ARG, "n_chunks out of range");
    std::vector<int32_t> sk, app, before;
    build_schedule(*cfg, n_chunks, sk, app, before);
    for (int64_t j = 0; j < n_chunks; ++j) {
      if (sinks) sinks[j] = sk[j];
      if (appends) appends[j] = app[j];
      if (rows) rows[j] = before[j] + sk[j] + app[j];
    }
    return KVM_OK;
  } catch (...) {
    return fail(KVM_E_INVALID_ARG, "host allocation failed");
  }
}

kvm_status kvm_state_create(const kvm_config* cfg, void* d_workspace, size_t workspace_bytes, void* stream,
                            kvm_state** out) {
  try {
    if (!out) return fail(KVM_E_INVALID_ARG, "out is NULL");
    *out = nullptr;
    Plan p;
    kvm_status s = plan(cfg, p);
    if (s != KVM_OK) return s;
    if (!d_workspace) return fail(KVM_E_INVALID_ARG, "workspace is NULL");
    if (!aligned(d_workspace, 256)) return fail(KVM_E_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < p.total)
      return fail(KVM_E_WORKSPACE, "workspace too small: need " + std::to_string(p.total) + " bytes");
    kvm_state* st = new (std::nothrow) kvm_state();
    if (!st) return fail(KVM_E_INVALID_ARG, "host allocation failed");
    st->cfg = *cfg;
    st->m = p.m;
    st->sched = std::move(p.sched);
    carve(p, reinterpret_cast<char*>(d_workspace), st->d);
    set_uniform(st);
    st->seqtab.assign((size_t)st->m.BH * kvm::kSeqFields, 0);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = clear_counters(st, true, hs);
    if (e == hipSuccess && !st->sched.empty())
      e = hipMemcpyAsync(st->d.sched, st->sched.data(), st->sched.size() * 4, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = kvm::launch_init(st->m, st->d, (double)cfg->rope_theta, hs);
    if (e != hipSuccess) {
      delete st;
      return fail(KVM_E_HIP, std::string("state initialisation: ") + hipGetErrorString(e));
    }
    *out = st;
    return KVM_OK;
  } catch (...) {
    return fail(KVM_E_INVALID_ARG, "host allocation failed");
  }
}

kvm_status kvm_state_destroy(kvm_state* st) {
  delete st;
  return KVM_OK;
}

kvm_status kvm_prefill(kvm_state* st, const void* q, const void* k, const void* v, const float* gate_logits, void* out,
                       int64_t n_tokens, void* stream) {
  if (!st) return fail(KVM_E_INVALID_ARG, "state is NULL");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  if (n_tokens < 0) return fail(KVM_E_INVALID_ARG, "n_tokens < 0");
  if (n_tokens == 0) return KVM_OK;
  if (!q || !k || !v || !gate_logits || !out) return fail(KVM_E_INVALID_ARG, "NULL tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(gate_logits, 4))
    return fail(KVM_E_INVALID_ARG, "tensors must be 16-byte aligned (gate logits 4-byte)");
  const kvm::Dims& m = st->m;
  if (st->per_seq) return fail(KVM_E_STATE, "sequences are at different positions: use kvm_prefill_ragged");
  if (st->pos % m.C != 0) return fail(KVM_E_STATE, "prefill must start at a multiple of chunk");
  if (st->pos + n_tokens > m.max_tokens) return fail(KVM_E_CAPACITY, "prefill would pass max_tokens");
  const size_t bytes = (size_t)m.BH * (size_t)n_tokens * 64 * (m.bf16 ? 2 : 4);
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
    return fail(KVM_E_INVALID_ARG, "out aliases an input");
  const int64_t p0 = st->pos, e = p0 + n_tokens;
  const int64_t c_first = p0 / m.C, c_last = (e - 1) / m.C;
  int64_t need = c_last - m.W / m.C;  // chunks the last query chunk needs absorbed
  if (need < 0) need = 0;
  const int64_t a1 = need > st->absorbed ? need : st->absorbed;
  if (a1 > m.J_cap) return fail(KVM_E_CAPACITY, "absorption would pass the workspace's chunk capacity");
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  kvm::Src src{q, k, v, gate_logits, p0, n_tokens};
  hipError_t err = hipSuccess;
  auto attn = [&](hipStream_t sx, int64_t cb, int64_t ce) {  // query chunks [cb, ce]
    const int s_max = rows_after(st, ce - m.W / m.C - 1);
    return timed(st, kAttn, sx,
                 [&] { return kvm::launch_attn(m, st->d, src, cb, (int)(ce - cb + 1), e, out, s_max, sx); });
  };
  auto rope = [&](hipStream_t sx) {
    if (!st->d.krot) return hipSuccess;
    return timed(st, kPrep, sx, [&] { return kvm::launch_rope_keys(m, st->d, src, sx); });
  };
  if (a1 > st->absorbed && (st->cfg.flags & KVM_FLAG_SERIAL_PREFILL)) {
    // every absorption first, then all the attention, on the caller's stream
    err = rope(hs);
    if (err == hipSuccess)
      err = timed(st, kScan, hs, [&] { return kvm::launch_scan(m, st->d, src, (int)st->absorbed, (int)a1, hs); });
    if (err == hipSuccess) err = attn(hs, c_first, c_last);
    if (err != hipSuccess) return hip_fail(st, err, "scan/attention launch");
  } else if (a1 > st->absorbed) {
    // Query chunk c reads the state after chunks [0, c - W/C) are absorbed.
    // Fork: the side stream starts after everything queued on hs so far.
    const int64_t wc = m.W / m.C;
    const std::vector<int64_t> pieces = scan_pieces(st->absorbed, a1);
    if (!st->side) err = hipStreamCreateWithFlags(&st->side, hipStreamNonBlocking);
    size_t ev = 0;
    hipEvent_t fork = err == hipSuccess ? sync_event(st, ev++) : nullptr;
    if (err == hipSuccess && !fork) err = hipErrorOutOfMemory;
    if (err == hipSuccess) err = hipEventRecord(fork, hs);
    if (err == hipSuccess) err = hipStreamWaitEvent(st->side, fork, 0);
    if (err == hipSuccess) err = rope(st->side);
    int64_t done = c_first - 1;  // attention queued through this chunk
    int64_t waited = st->absorbed;   // chunks absorbed before the side stream's last wait
    // The ring fill overwrites the slots of the tokens before p0: the scan reads
    // them for chunks below c_first and the attention for query chunks through
    // c_ring.  Once both are behind the side stream it goes there, beside the
    // remaining pieces, instead of after the join.
    const int64_t c_ring = std::min(c_last, c_first + wc - 1);
    const int64_t from = e - m.R > p0 ? e - m.R : p0;
    bool ring_queued = false;
    auto ring_side = [&] {
      if (!ring_queued && err == hipSuccess && waited >= c_first && done >= c_ring) {
        err = timed(st, kRing, st->side, [&] { return kvm::launch_ring_fill(m, st->d, src, from, e, st->side); });
        ring_queued = true;
      }
    };
    auto release = [&](int64_t absorbed) {
      const int64_t hi = std::min(c_last, absorbed + wc);
      if (err == hipSuccess && hi > done) {
        err = attn(st->side, done + 1, hi);
        done = hi;
      }
    };
    release(pieces.front());
    ring_side();
    for (size_t i = 0; i + 1 < pieces.size() && err == hipSuccess; ++i) {
      const int64_t jb = pieces[i], je = pieces[i + 1];
      err = timed(st, kScan, hs, [&] { return kvm::launch_scan(m, st->d, src, (int)jb, (int)je, hs); });
      if (err == hipSuccess && done < c_last) {
        hipEvent_t ready = sync_event(st, ev++);
        if (!ready) err = hipErrorOutOfMemory;
        if (err == hipSuccess) err = hipEventRecord(ready, hs);
        if (err == hipSuccess) err = hipStreamWaitEvent(st->side, ready, 0);
        if (err == hipSuccess) waited = je;
        release(je);
      }
      ring_side();
    }
    // Join: hs continues only after the side stream's attention.
    hipEvent_t join = err == hipSuccess ? sync_event(st, ev++) : nullptr;
    if (err == hipSuccess && !join) err = hipErrorOutOfMemory;
    if (err == hipSuccess) err = hipEventRecord(join, st->side);
    if (err == hipSuccess) err = hipStreamWaitEvent(hs, join, 0);
    if (err == hipSuccess && done != c_last) err = hipErrorInvalidValue;
    if (err == hipSuccess && !ring_queued)
      err = timed(st, kRing, hs, [&] { return kvm::launch_ring_fill(m, st->d, src, from, e, hs); });
    if (err != hipSuccess) return hip_fail(st, err, "scan/attention/ring launch");
  } else {
    err = rope(hs);
    if (err == hipSuccess) err = attn(hs, c_first, c_last);
    if (err != hipSuccess) return hip_fail(st, err, "attention launch");
  }
  if (!(a1 > st->absorbed) || (st->cfg.flags & KVM_FLAG_SERIAL_PREFILL)) {
    const int64_t from = e - m.R > p0 ? e - m.R : p0;
    err = timed(st, kRing, hs, [&] { return kvm::launch_ring_fill(m, st->d, src, from, e, hs); });
    if (err != hipSuccess) return hip_fail(st, err, "ring launch");
  }
  st->pos = e;
  st->absorbed = a1;
  set_uniform(st);
  return KVM_OK;
}

kvm_status kvm_prefill_noalloc(const kvm_config* cfg, const void* q, const void* k, const void* v,
                               const float* gate_logits, void* out, int64_t n_tokens, void* stream) {
  // No device or host allocation on the success path: the plan keeps no
  // schedule vector, the schedule table is computed on the device, counters are
  // cleared by a fill kernel, and the workspace is the static scratch.
  Plan p;
  kvm_status s = plan(cfg, p, false);
  if (s != KVM_OK) return s;
  if (cfg->flags & KVM_FLAG_TRACE) return fail(KVM_E_INVALID_ARG, "KVM_FLAG_TRACE needs a state to read the trace from");
  if (cfg->sched == KVM_SCHED_POWER)
    return fail(KVM_E_INVALID_ARG, "the power schedule is not available here (the device builds integer schedules only)");
  if (p.total > kvm::kScratchBytes)
    return fail(KVM_E_WORKSPACE, "the configuration needs " + std::to_string(p.total) +
                                     " bytes of workspace; the static scratch holds " + std::to_string(kvm::kScratchBytes));
  if (n_tokens < 0 || n_tokens > cfg->max_tokens) return fail(KVM_E_INVALID_ARG, "n_tokens must be in [0, max_tokens]");
  if (n_tokens == 0) return KVM_OK;
  if (!q || !k || !v || !gate_logits || !out) return fail(KVM_E_INVALID_ARG, "NULL tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(gate_logits, 4))
    return fail(KVM_E_INVALID_ARG, "tensors must be 16-byte aligned (gate logits 4-byte)");
  const kvm::Dims& m = p.m;
  const size_t bytes = (size_t)m.BH * (size_t)n_tokens * 64 * (m.bf16 ? 2 : 4);
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
    return fail(KVM_E_INVALID_ARG, "out aliases an input");
  void* base = nullptr;
  hipError_t err = kvm::scratch_address(&base);
  if (err != hipSuccess) return fail(KVM_E_HIP, std::string("scratch address: ") + hipGetErrorString(err));
  kvm::Dev d{};
  carve(p, reinterpret_cast<char*>(base), d);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int64_t c_last = (n_tokens - 1) / m.C;
  const int64_t a1 = std::max<int64_t>(0, c_last - m.W / m.C);   // chunks the last query chunk needs
  int s_max = 0;                                                 // rows of the last snapshot read
  for_each_chunk(*cfg, a1, [&](int64_t, int32_t sk, int32_t app, int32_t before) { s_max = before + sk + app; });
  const kvm::SchedParams sp{m.C, m.ns, cfg->sched, cfg->max_slots, cfg->alpha, m.J_cap};
  kvm::Src src{q, k, v, gate_logits, 0, n_tokens};
  err = kvm::launch_noalloc_init(m, d, sp, (double)cfg->rope_theta, hs);
  if (err == hipSuccess && d.krot) err = kvm::launch_rope_keys(m, d, src, hs);
  if (err == hipSuccess) err = kvm::launch_scan(m, d, src, 0, (int)a1, hs);
  if (err == hipSuccess) err = kvm::launch_attn(m, d, src, 0, (int)(c_last + 1), n_tokens, out, s_max, hs);
  if (err != hipSuccess) return fail(KVM_E_HIP, std::string("prefill launch: ") + hipGetErrorString(err));
  return KVM_OK;
}

kvm_status kvm_decode_step(kvm_state* st, const void* q, const void* k, const void* v, const float* gate_logits,
                           void* out, void* stream) {
  if (!st) return fail(KVM_E_INVALID_ARG, "state is NULL");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  if (!q || !k || !v || !gate_logits || !out) return fail(KVM_E_INVALID_ARG, "NULL tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(gate_logits, 4))
    return fail(KVM_E_INVALID_ARG, "tensors must be 16-byte aligned (gate logits 4-byte)");
  const kvm::Dims& m = st->m;
  if (st->per_seq) return fail(KVM_E_STATE, "sequences are at different positions: use kvm_decode_step_ragged");
  const int64_t t = st->pos;
  if (t + 1 > m.max_tokens) return fail(KVM_E_CAPACITY, "decode would pass max_tokens");
  const size_t bytes = (size_t)m.BH * 64 * (m.bf16 ? 2 : 4);
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
    return fail(KVM_E_INVALID_ARG, "out aliases an input");
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  int64_t absorbed = st->absorbed;
  if (t % m.C == 0 && t >= m.W + m.C) {
    const int64_t j = (t - m.W - m.C) / m.C;
    if (j != absorbed || j >= m.J_cap) return fail(KVM_E_STATE, "absorbed chunk count out of step with position");
    kvm::Src src{nullptr, nullptr, nullptr, nullptr, t, 0};  // every position < t comes from the ring
    hipError_t err = timed(st, kDecAbsorb, hs, [&] { return kvm::launch_scan(m, st->d, src, (int)j, (int)j + 1, hs); });
    if (err != hipSuccess) return hip_fail(st, err, "decode absorb launch");
    absorbed = j + 1;
  }
  const int rows = rows_after(st, absorbed - 1);
  hipError_t err = timed(st, kDecAttn, hs, [&] {
    return kvm::launch_decode(m, st->d, q, k, v, gate_logits, t, rows, out, hs);
  });
  if (err != hipSuccess) return hip_fail(st, err, "decode launch");
  st->pos = t + 1;
  st->absorbed = absorbed;
  set_uniform(st);
  return KVM_OK;
}

namespace {
struct BwdPlan {
  size_t part_win, part_state, tot_rho, lse_d, qr32, kr32, total;
};
BwdPlan bwd_plan(const kvm::Dims& m, int64_t n_tokens) {
  BwdPlan b{};
  const size_t BH = (size_t)m.BH;
  const size_t nq = (size_t)((n_tokens + m.C - 1) / m.C);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  b.part_win = take(BH * nq * (size_t)m.R * 128 * 4);
  b.part_state = take(BH * (size_t)m.idx_total * 96 * 4);
  b.tot_rho = take(BH * (size_t)m.idx_total * 4);
  b.lse_d = take(BH * (size_t)n_tokens * 8);
  b.qr32 = take(BH * (size_t)n_tokens * 64 * 4);
  b.kr32 = take(BH * (size_t)n_tokens * 64 * 4);
  b.total = off;
  return b;
}
}  // namespace

kvm_status kvm_backward_workspace_bytes(const kvm_config* cfg, size_t* bytes) {
  try {
    if (!bytes) return fail(KVM_E_INVALID_ARG, "bytes is NULL");
    Plan p;
    kvm_status s = plan(cfg, p, false);
    if (s != KVM_OK) return s;
    *bytes = bwd_plan(p.m, cfg->max_tokens).total;
    return KVM_OK;
  } catch (...) {
    return fail(KVM_E_INVALID_ARG, "host allocation failed");
  }
}

kvm_status kvm_prefill_backward(kvm_state* st, const void* q, const void* k, const void* v, const float* gate_logits,
                                const void* d_out, float* d_q, float* d_k, float* d_v, float* d_gate,
                                int64_t n_tokens, void* d_workspace, size_t workspace_bytes, void* stream) {
  if (!st) return fail(KVM_E_INVALID_ARG, "state is NULL");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  const kvm::Dims& m = st->m;
  if (!m.trace) return fail(KVM_E_INVALID_ARG, "the backward reads the forward's decisions: create the state with KVM_FLAG_TRACE");
  if (n_tokens <= 0) return fail(KVM_E_INVALID_ARG, "n_tokens must be > 0");
  if (st->per_seq) return fail(KVM_E_STATE, "sequences are at different positions");
  if (n_tokens != st->pos) return fail(KVM_E_STATE, "the state's position must equal n_tokens");
  if (!q || !k || !v || !gate_logits || !d_out || !d_q || !d_k || !d_v || !d_gate || !d_workspace)
    return fail(KVM_E_INVALID_ARG, "NULL pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_out, 16) || !aligned(d_q, 16) ||
      !aligned(d_k, 16) || !aligned(d_v, 16) || !aligned(gate_logits, 4) || !aligned(d_gate, 4))
    return fail(KVM_E_INVALID_ARG, "tensors must be 16-byte aligned (gate logits 4-byte)");
  if (!aligned(d_workspace, 256)) return fail(KVM_E_WORKSPACE, "workspace must be 256-byte aligned");
  const BwdPlan bp = bwd_plan(m, n_tokens);
  if (workspace_bytes < bp.total)
    return fail(KVM_E_WORKSPACE, "backward workspace too small: need " + std::to_string(bp.total) + " bytes");
  char* w = reinterpret_cast<char*>(d_workspace);
  kvm::Bwd b{};
  b.part_win = reinterpret_cast<float*>(w + bp.part_win);
  b.part_state = reinterpret_cast<float*>(w + bp.part_state);
  b.tot_rho = reinterpret_cast<float*>(w + bp.tot_rho);
  b.lse_d = reinterpret_cast<float2*>(w + bp.lse_d);
  b.qr32 = reinterpret_cast<float*>(w + bp.qr32);
  b.kr32 = reinterpret_cast<float*>(w + bp.kr32);
  b.dq = d_q;
  b.dk = d_k;
  b.dv = d_v;
  b.dl = d_gate;
  b.nq = (int)((n_tokens + m.C - 1) / m.C);
  b.absorbed = (int)st->absorbed;
  const kvm::BwdIn in{q, k, v, gate_logits, d_out, n_tokens};
  const int rows_last = rows_after(st, st->absorbed - 1);
  hipError_t e = kvm::launch_backward(m, st->d, in, b, rows_last, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(st, e, "backward launch");
  return KVM_OK;
}

kvm_status kvm_project_in(const kvm_config* cfg, const void* x, const void* w_in, const float* b_gate, void* q,
                          void* k, void* v, float* gate_logits, int64_t n_tokens, void* stream) {
  kvm_status s = validate(cfg);
  if (s != KVM_OK) return s;
  if (n_tokens < 0 || n_tokens > ((int64_t)1 << 31)) return fail(KVM_E_INVALID_ARG, "n_tokens out of range");
  if (n_tokens == 0) return KVM_OK;
  if (!x || !w_in || !q || !k || !v || !gate_logits) return fail(KVM_E_INVALID_ARG, "NULL pointer");
  if (!aligned(x, 16) || !aligned(w_in, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(gate_logits, 4) || (b_gate && !aligned(b_gate, 4)))
    return fail(KVM_E_INVALID_ARG, "tensors must be 16-byte aligned (gate logits and bias 4-byte)");
  kvm::ProjArgs a{};
  a.x = x;
  a.w = w_in;
  a.bias = b_gate;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gl = gate_logits;
  a.H = cfg->heads;
  a.K = cfg->heads * 64;
  a.Nout = 3 * a.K + a.H;
  a.N = n_tokens;
  a.M = (int64_t)cfg->batch * n_tokens;
  hipError_t e = kvm::launch_proj(a, false, cfg->dtype == KVM_BF16, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVM_E_HIP, std::string("projection launch: ") + hipGetErrorString(e));
  return KVM_OK;
}

kvm_status kvm_project_out(const kvm_config* cfg, const void* o, const void* w_out, void* y, int64_t n_tokens,
                           void* stream) {
  kvm_status s = validate(cfg);
  if (s != KVM_OK) return s;
  if (n_tokens < 0 || n_tokens > ((int64_t)1 << 31)) return fail(KVM_E_INVALID_ARG, "n_tokens out of range");
  if (n_tokens == 0) return KVM_OK;
  if (!o || !w_out || !y) return fail(KVM_E_INVALID_ARG, "NULL pointer");
  if (!aligned(o, 16) || !aligned(w_out, 16) || !aligned(y, 16))
    return fail(KVM_E_INVALID_ARG, "tensors must be 16-byte aligned");
  kvm::ProjArgs a{};
  a.x = o;
  a.w = w_out;
  a.y = y;
  a.H = cfg->heads;
  a.K = cfg->heads * 64;
  a.Nout = a.K;
  a.N = n_tokens;
  a.M = (int64_t)cfg->batch * n_tokens;
  hipError_t e = kvm::launch_proj(a, true, cfg->dtype == KVM_BF16, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVM_E_HIP, std::string("projection launch: ") + hipGetErrorString(e));
  return KVM_OK;
}

kvm_status kvm_state_read(const kvm_state* st, int64_t chunk, kvm_state_view* dst, void* stream) {
  if (!st || !dst) return fail(KVM_E_INVALID_ARG, "NULL argument");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  const kvm::Dims& m = st->m;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const size_t BH = (size_t)m.BH, S = (size_t)m.S_cap, es = m.bf16 ? 2 : 4;
  const int64_t min_abs = *std::min_element(st->sabs.begin(), st->sabs.end());
  if (chunk < -1 || chunk >= min_abs)
    return fail(KVM_E_INVALID_ARG, "chunk must be -1 (current state) or a chunk every sequence has absorbed");
  if (chunk >= 0) {
    // a past snapshot: read-form row versions only
    if (dst->key_sum || dst->val_sum || dst->ring_k || dst->ring_v || dst->ring_l || dst->trace_slot ||
        dst->trace_kind)
      return fail(KVM_E_INVALID_ARG,
                  "a past snapshot keeps only read-form row versions: raw sums, ring and trace are current-state only");
    const int rows = rows_after(st, chunk);
    const int64_t ioff = st->sched[(size_t)chunk * 4 + 3];
    hipError_t e = kvm::launch_snapshot_gather(m, st->d, rows, ioff, m.S_cap, dst->key_read, dst->val_read, dst->rho,
                                               dst->count, hs);
    if (e != hipSuccess) return hip_fail(const_cast<kvm_state*>(st), e, "snapshot gather launch");
    if (dst->n_rows)
      for (size_t s = 0; s < BH; ++s) dst->n_rows[s] = rows;
    return KVM_OK;
  }
  if ((dst->trace_slot || dst->trace_kind) && !m.trace)
    return fail(KVM_E_INVALID_ARG, "trace requested but the state was created without KVM_FLAG_TRACE");
  struct Copy {
    void* to;
    const void* from;
    size_t bytes;
  } copies[] = {
      {dst->key_sum, st->d.key_sum, BH * S * 32 * 4},
      {dst->val_sum, st->d.val_sum, BH * S * 64 * 4},
      {dst->count, st->d.count, BH * S * 4},
      {dst->rho, st->d.rho, BH * S * 4},
      {dst->key_read, st->d.kread, BH * S * 32 * es},
      {dst->val_read, st->d.vread, BH * S * 64 * es},
      {dst->trace_slot, st->d.tslot, BH * (size_t)m.max_tokens * 4},
      {dst->trace_kind, st->d.tkind, BH * (size_t)m.max_tokens},
      {dst->ring_k, st->d.ring_k, BH * (size_t)m.R * 64 * es},
      {dst->ring_v, st->d.ring_v, BH * (size_t)m.R * 64 * es},
      {dst->ring_l, st->d.ring_l, BH * (size_t)m.R * 4},
  };
  for (const Copy& c : copies) {
    if (!c.to || c.bytes == 0) continue;
    hipError_t e = hipMemcpyAsync(c.to, c.from, c.bytes, hipMemcpyDefault, hs);
    if (e != hipSuccess) return hip_fail(const_cast<kvm_state*>(st), e, "state copy");
  }
  if (dst->n_rows)   // host memory: the row count is host-side
    for (size_t s = 0; s < BH; ++s) dst->n_rows[s] = rows_after(st, st->sabs[s] - 1);
  dst->position = st->per_seq ? -1 : st->pos;
  return KVM_OK;
}

kvm_status kvm_state_load(kvm_state* st, const kvm_state_view* src, void* stream) {
  if (!st || !src) return fail(KVM_E_INVALID_ARG, "NULL argument");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  const kvm::Dims& m = st->m;
  const int64_t pos = src->position;
  if (pos < 0 || pos > m.max_tokens) return fail(KVM_E_INVALID_ARG, "position outside [0, max_tokens]");
  const int64_t absorbed = absorbed_at(m, pos);
  if (absorbed > m.J_cap) return fail(KVM_E_INVALID_ARG, "position needs more absorbed chunks than the workspace holds");
  const int rows = rows_after(st, absorbed - 1);
  const size_t BH = (size_t)m.BH, S = (size_t)m.S_cap, es = m.bf16 ? 2 : 4;
  if (src->n_rows)
    for (size_t s = 0; s < BH; ++s)
      if (src->n_rows[s] != rows)
        return fail(KVM_E_INVALID_ARG, "n_rows[" + std::to_string(s) + "] = " + std::to_string(src->n_rows[s]) +
                                           " but the schedule has " + std::to_string(rows) + " rows at this position");
  if (rows > 0 && (!src->key_sum || !src->val_sum || !src->count || !src->rho))
    return fail(KVM_E_INVALID_ARG, "key_sum, val_sum, count and rho are required when the state has rows");
  if (pos > 0 && (!src->ring_k || !src->ring_v || !src->ring_l))
    return fail(KVM_E_INVALID_ARG, "ring_k, ring_v and ring_l are required when position > 0");
  if ((src->trace_slot || src->trace_kind) && !m.trace)
    return fail(KVM_E_INVALID_ARG, "trace given but the state was created without KVM_FLAG_TRACE");
  if (m.trace && (!src->trace_slot != !src->trace_kind))
    return fail(KVM_E_INVALID_ARG, "give both trace arrays or neither");
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = clear_counters(st, !src->trace_slot, hs);
  struct Copy {
    void* to;
    const void* from;
    size_t bytes;
  } copies[] = {
      {st->d.key_sum, src->key_sum, BH * S * 32 * 4},
      {st->d.val_sum, src->val_sum, BH * S * 64 * 4},
      {st->d.count, src->count, BH * S * 4},
      {st->d.rho, src->rho, BH * S * 4},
      {st->d.ring_k, src->ring_k, BH * (size_t)m.R * 64 * es},
      {st->d.ring_v, src->ring_v, BH * (size_t)m.R * 64 * es},
      {st->d.ring_l, src->ring_l, BH * (size_t)m.R * 4},
      {st->d.tslot, src->trace_slot, BH * (size_t)m.max_tokens * 4},
      {st->d.tkind, src->trace_kind, BH * (size_t)m.max_tokens},
  };
  for (const Copy& c : copies) {
    if (e != hipSuccess) break;
    if (!c.from || c.bytes == 0) continue;
    e = hipMemcpyAsync(c.to, c.from, c.bytes, hipMemcpyDefault, hs);
  }
  if (e == hipSuccess && rows > 0)
    e = kvm::launch_state_load(m, st->d, rows, absorbed > 0 ? st->sched[(size_t)(absorbed - 1) * 4 + 3] : -1, hs);
  if (e != hipSuccess) return hip_fail(st, e, "state load");
  st->pos = pos;
  st->absorbed = absorbed;
  set_uniform(st);
  return KVM_OK;
}

kvm_status kvm_snapshot_read(const kvm_state* st, int64_t j, void* key_read, void* val_read, float* rho_read,
                             void* stream) {
  if (!st) return fail(KVM_E_INVALID_ARG, "state is NULL");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  if (j < 0 || j >= *std::min_element(st->sabs.begin(), st->sabs.end()))
    return fail(KVM_E_INVALID_ARG, "chunk j has not been absorbed by every sequence");
  const int rows = rows_after(st, j);
  const int64_t ioff = st->sched[(size_t)j * 4 + 3];
  hipError_t e = kvm::launch_snapshot_gather(st->m, st->d, rows, ioff, rows, key_read, val_read, rho_read, nullptr,
                                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(const_cast<kvm_state*>(st), e, "snapshot gather launch");
  return KVM_OK;
}

kvm_status kvm_state_positions(const kvm_state* st, int64_t* positions) {
  if (!st || !positions) return fail(KVM_E_INVALID_ARG, "NULL argument");
  for (size_t s = 0; s < st->spos.size(); ++s) positions[s] = st->spos[s];
  return KVM_OK;
}

kvm_status kvm_state_reset_sequence(kvm_state* st, int32_t seq, void* stream) {
  if (!st) return fail(KVM_E_INVALID_ARG, "state is NULL");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  if (seq < 0 || seq >= st->m.BH) return fail(KVM_E_INVALID_ARG, "sequence index out of range");
  hipError_t e = kvm::launch_seq_reset(st->m, st->d, seq, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(st, e, "sequence reset");
  st->spos[(size_t)seq] = 0;
  st->sabs[(size_t)seq] = 0;
  sync_uniform(st);
  return KVM_OK;
}

kvm_status kvm_prefill_ragged(kvm_state* st, const int64_t* n_tokens, const void* q, const void* k, const void* v,
                              const float* gate_logits, void* out, int64_t n_max, void* stream) {
  if (!st || !n_tokens) return fail(KVM_E_INVALID_ARG, "NULL argument");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  if (n_max < 0) return fail(KVM_E_INVALID_ARG, "n_max < 0");
  const kvm::Dims& m = st->m;
  const size_t BH = (size_t)m.BH;
  // per sequence: its own range of positions, chunks to absorb and query chunks
  int64_t nq_max = 0, span_max = 0, any_abs = 0;
  int s_max = 0;
  std::vector<int64_t>& tab = st->seqtab;
  std::fill(tab.begin(), tab.end(), 0);
  for (size_t s = 0; s < BH; ++s) {
    const int64_t n = n_tokens[s], p0 = st->spos[s];
    if (n < 0 || n > n_max) return fail(KVM_E_INVALID_ARG, "n_tokens[s] must be in [0, n_max]");
    int64_t* r = &tab[s * kvm::kSeqFields];
    r[kvm::kSeqP0] = p0;
    r[kvm::kSeqJb] = r[kvm::kSeqJe] = st->sabs[s];
    if (n == 0) continue;
    if (p0 % m.C != 0) return fail(KVM_E_STATE, "sequence " + std::to_string(s) + ": prefill must start at a multiple of chunk");
    const int64_t e = p0 + n;
    if (e > m.max_tokens) return fail(KVM_E_CAPACITY, "sequence " + std::to_string(s) + ": prefill would pass max_tokens");
    const int64_t c_first = p0 / m.C, c_last = (e - 1) / m.C;
    int64_t need = c_last - m.W / m.C;
    if (need < 0) need = 0;
    const int64_t a1 = std::max(need, st->sabs[s]);
    if (a1 > m.J_cap) return fail(KVM_E_CAPACITY, "absorption would pass the workspace's chunk capacity");
    r[kvm::kSeqJe] = a1;
    r[kvm::kSeqCb] = c_first;
    r[kvm::kSeqNq] = c_last - c_first + 1;
    r[kvm::kSeqEnd] = e;
    r[kvm::kSeqN] = n;
    r[kvm::kSeqFrom] = std::max(e - m.R, p0);
    r[kvm::kSeqTo] = e;
    nq_max = std::max(nq_max, c_last - c_first + 1);
    span_max = std::max(span_max, e - r[kvm::kSeqFrom]);
    any_abs |= a1 > st->sabs[s];
    s_max = std::max(s_max, rows_after(st, c_last - m.W / m.C - 1));
  }
  if (nq_max == 0) return KVM_OK;
  if (!q || !k || !v || !gate_logits || !out) return fail(KVM_E_INVALID_ARG, "NULL tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(gate_logits, 4))
    return fail(KVM_E_INVALID_ARG, "tensors must be 16-byte aligned (gate logits 4-byte)");
  const size_t bytes = BH * (size_t)n_max * 64 * (m.bf16 ? 2 : 4);
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
    return fail(KVM_E_INVALID_ARG, "out aliases an input");
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  kvm::Src src{q, k, v, gate_logits, 0, n_max, st->d.seq};
  hipError_t err = upload_seq(st, hs);
  if (err == hipSuccess && st->d.krot) err = timed(st, kPrep, hs, [&] { return kvm::launch_rope_keys(m, st->d, src, hs); });
  if (err == hipSuccess && any_abs)
    err = timed(st, kScan, hs, [&] { return kvm::launch_scan(m, st->d, src, 0, 1, hs); });
  if (err == hipSuccess)
    err = timed(st, kAttn, hs, [&] { return kvm::launch_attn(m, st->d, src, 0, (int)nq_max, 0, out, s_max, hs); });
  if (err == hipSuccess)
    err = timed(st, kRing, hs, [&] { return kvm::launch_ring_fill(m, st->d, src, 0, span_max, hs); });
  if (err != hipSuccess) return hip_fail(st, err, "ragged prefill launch");
  for (size_t s = 0; s < BH; ++s) {
    const int64_t* r = &tab[s * kvm::kSeqFields];
    if (n_tokens[s] == 0) continue;
    st->spos[s] = r[kvm::kSeqEnd];
    st->sabs[s] = r[kvm::kSeqJe];
  }
  sync_uniform(st);
  return KVM_OK;
}

kvm_status kvm_decode_step_ragged(kvm_state* st, const uint8_t* active, const void* q, const void* k, const void* v,
                                  const float* gate_logits, void* out, void* stream) {
  if (!st || !active) return fail(KVM_E_INVALID_ARG, "NULL argument");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  if (!q || !k || !v || !gate_logits || !out) return fail(KVM_E_INVALID_ARG, "NULL tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(gate_logits, 4))
    return fail(KVM_E_INVALID_ARG, "tensors must be 16-byte aligned (gate logits 4-byte)");
  const kvm::Dims& m = st->m;
  const size_t BH = (size_t)m.BH;
  const size_t bytes = BH * 64 * (m.bf16 ? 2 : 4);
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
    return fail(KVM_E_INVALID_ARG, "out aliases an input");
  std::vector<int64_t>& tab = st->seqtab;
  std::fill(tab.begin(), tab.end(), 0);
  bool any = false, any_abs = false;
  for (size_t s = 0; s < BH; ++s) {
    int64_t* r = &tab[s * kvm::kSeqFields];
    r[kvm::kSeqP0] = INT64_MAX;    // every token an absorption reads comes from the ring
    if (!active[s]) continue;
    const int64_t t = st->spos[s];
    if (t + 1 > m.max_tokens) return fail(KVM_E_CAPACITY, "sequence " + std::to_string(s) + ": decode would pass max_tokens");
    r[kvm::kSeqActive] = 1;
    r[kvm::kSeqPos] = t;
    any = true;
    if (t % m.C == 0 && t >= m.W + m.C) {
      const int64_t j = (t - m.W - m.C) / m.C;
      if (j != st->sabs[s] || j >= m.J_cap) return fail(KVM_E_STATE, "absorbed chunk count out of step with position");
      r[kvm::kSeqJb] = j;
      r[kvm::kSeqJe] = j + 1;
      any_abs = true;
    }
  }
  if (!any) return KVM_OK;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  kvm::Src src{nullptr, nullptr, nullptr, nullptr, 0, 0, st->d.seq};
  hipError_t err = upload_seq(st, hs);
  if (err == hipSuccess && any_abs)
    err = timed(st, kDecAbsorb, hs, [&] { return kvm::launch_scan(m, st->d, src, 0, 1, hs); });
  if (err == hipSuccess)
    err = timed(st, kDecAttn, hs,
                [&] { return kvm::launch_decode(m, st->d, q, k, v, gate_logits, 0, 0, out, hs, st->d.seq); });
  if (err != hipSuccess) return hip_fail(st, err, "ragged decode launch");
  for (size_t s = 0; s < BH; ++s) {
    if (!active[s]) continue;
    const int64_t* r = &tab[s * kvm::kSeqFields];
    if (r[kvm::kSeqJe] > r[kvm::kSeqJb]) st->sabs[s] = r[kvm::kSeqJe];
    st->spos[s] += 1;
  }
  sync_uniform(st);
  return KVM_OK;
}

kvm_status kvm_state_get_info(const kvm_state* st, kvm_state_info* info) {
  if (!st || !info) return fail(KVM_E_INVALID_ARG, "NULL argument");
  info->position = st->per_seq ? -1 : st->pos;
  info->absorbed_chunks = st->per_seq ? -1 : st->absorbed;
  info->rows = st->per_seq ? -1 : rows_after(st, st->absorbed - 1);
  info->per_sequence = st->per_seq ? 1 : 0;
  info->max_rows = st->m.S_cap;
  info->max_chunks = st->m.J_cap;
  info->poisoned = st->poisoned ? 1 : 0;
  info->scan_groups = st->m.P;
  return KVM_OK;
}

kvm_status kvm_state_check(kvm_state* st, void* stream) {
  if (!st) return fail(KVM_E_INVALID_ARG, "state is NULL");
  if (st->poisoned) return fail(KVM_E_STATE, "state is poisoned by an earlier HIP failure");
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  int flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, st->d.xerr, 4, hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_fail(st, e, "state check");
  if (flag != 0) {
    st->poisoned = true;
    return fail(KVM_E_HIP, "an absorption scan workgroup gave up waiting at a cross-workgroup exchange");
  }
  return KVM_OK;
}

kvm_status kvm_state_reset(kvm_state* st, void* stream) {
  if (!st) return fail(KVM_E_INVALID_ARG, "state is NULL");
  hipError_t e = clear_counters(st, true, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(st, e, "state reset");
  st->pos = 0;
  st->absorbed = 0;
  set_uniform(st);
  st->poisoned = false;
  return KVM_OK;
}

kvm_status kvm_profile_enable(kvm_state* st, int phases) {
  if (!st) return fail(KVM_E_INVALID_ARG, "state is NULL");
  if (phases & ~KVM_PROFILE_ALL) return fail(KVM_E_INVALID_ARG, "unknown profile phase bits");
  st->profiling = phases;
  return KVM_OK;
}

kvm_status kvm_profile_read(kvm_state* st, kvm_profile_times* out) {
  if (!st || !out) return fail(KVM_E_INVALID_ARG, "NULL argument");
  double ms[kPhases] = {0};
  int64_t n[kPhases] = {0};
  hipError_t err = hipSuccess;
  for (kvm_state::Rec& r : st->recs) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e == hipSuccess) {
      ms[r.phase] += t;
      n[r.phase] += 1;
    } else if (err == hipSuccess) {
      err = e;
    }
    st->pool.push_back(r.a);
    st->pool.push_back(r.b);
  }
  st->recs.clear();
  out->scan_ms = ms[kScan];
  out->scan_launches = n[kScan];
  out->attn_ms = ms[kAttn];
  out->attn_launches = n[kAttn];
  out->ring_ms = ms[kRing];
  out->ring_launches = n[kRing];
  out->dec_absorb_ms = ms[kDecAbsorb];
  out->dec_absorb_launches = n[kDecAbsorb];
  out->dec_attn_ms = ms[kDecAttn];
  out->dec_attn_launches = n[kDecAttn];
  out->prep_ms = ms[kPrep];
  out->prep_launches = n[kPrep];
  if (err != hipSuccess) return fail(KVM_E_HIP, std::string("profile events: ") + hipGetErrorString(err));
  return KVM_OK;
}

const char* kvm_status_str(kvm_status s) {
  switch (s) {
    case KVM_OK: return "KVM_OK";
    case KVM_E_INVALID_ARG: return "KVM_E_INVALID_ARG";
    case KVM_E_WORKSPACE: return "KVM_E_WORKSPACE";
    case KVM_E_CAPACITY: return "KVM_E_CAPACITY";
    case KVM_E_STATE: return "KVM_E_STATE";
    case KVM_E_HIP: return "KVM_E_HIP";
  }
  return "KVM_E_UNKNOWN";
}

const char* kvm_last_error(void) { return g_err.c_str(); }

}  // extern "C"
