// Scheduling rules of the persistent forward (persistent.hip), written once and compiled
// twice: into the device kernel, and into a host-threaded model of that kernel that the
// CPU test suite runs (one host thread per workgroup, the same rules, random timing).
// Nothing here touches memory directly: control words are read and claimed through an
// `Ops` object (device atomics on the GPU, std::atomic in the model).
//
// What the rules encode (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del
// 2.37x ...", section 02: communication and compute parts of one kernel notify each other
// through GPU-local counters, tokens reach the experts one minibatch at a time through a
// fixed ring of slots that are reused right after combine; qubstore.ru "Смесь котят ...",
// ring buffer paragraph):
// * Pipelines.  The row tiles (256 rows of one expert) are split into n_part contiguous,
//   balanced ranges; pipeline p owns [lo, hi) with its own ring partition of S slots and
//   its own counters.
// * Chunks and slots.  A row tile is cpm chunks (one minibatch of 256 / cpm rows each).
//   Pipeline-local chunk q lives in slot q mod S; it may be gathered once the previous
//   occupant (chunk q - S) has been pushed, i.e. once the slot's epoch counter, bumped by
//   every push, reaches q / S.
// * Groups.  Consecutive row tiles of one expert, at most G of them, form a group.  The
//   gate/up phase U(g) of group g runs its tiles column-panel-major (all row tiles of the
//   group for weight panel 0, then panel 1, ...), so the workgroups that run at the same
//   time share one weight panel; the down phase D(g) likewise.
// * Ticket order.  With look-ahead (the ring holds at least two groups): U0, U1, D0, U2, D1, ...,
//   U(n-1), D(n-2), D(n-1); without: U0, D0, U1, D1, ...  A task waits only for gathers
//   or for tasks with smaller tickets, and a gather waits only for a push, which waits
//   only for tasks with smaller tickets than any task that waits for that gather, so the
//   smallest unfinished ticket can always run: no deadlock, whatever the timing.
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define MOE_HD __host__ __device__ inline
#else
#define MOE_HD inline
#endif

namespace moe {
namespace sched {

constexpr int kMaxPipes = 8;
constexpr int kMaxGroup = 8;          // row tiles per group, at most
constexpr int kPipeWords = 16;        // control words per pipeline

// per-pipeline control words (offsets inside a pipeline's 16 words)
enum PipeWord {
  kJoin = 0,        // workgroups that joined (arrival order = rank)
  kGatherNext = 1,  // next chunk to claim for gathering
  kPushNext = 2,    // next chunk to claim for pushing
  kTicketNext = 3,  // next compute ticket
  kNGroups = 4,     // groups (written by the preparation kernel)
  kNTickets = 5,    // compute tasks
  kLo = 6,          // first row tile
  kHi = 7,          // one past the last row tile
};

// Word offsets of the control block (int32 words, zeroed before every launch).
struct CtrlLayout {
  int abort_word;    // set by a watchdog expiry: every loop exits
  int pipe0;         // kMaxPipes x kPipeWords
  int filled;        // [max_mtiles * 4]: chunk h of row tile m gathered (m * 4 + h)
  int g1_done;       // [max_mtiles]: gate/up tiles of row tile m finished
  int g2_done;       // [max_mtiles]: down tiles of row tile m finished
  int grp_first;     // [max_mtiles]: group tables, pipeline p's groups from index lo
  int grp_len;       // [max_mtiles]
  int phase_start;   // [2 * max_mtiles + kMaxPipes]: pipeline p's phases from 2 lo + p
  int slot_epoch;    // [max_slots]: pushes that freed the slot
  int resident;      // [max_mtiles * 4]: after a reverse-ring launch, 1 + the ring slot that
                     // still holds chunk h of row tile m (m * 4 + h), or 0
  int words;         // total
};

MOE_HD CtrlLayout ctrl_layout(int max_mtiles, int max_slots) {
  CtrlLayout c;
  c.abort_word = 0;
  c.pipe0 = 16;
  c.filled = c.pipe0 + kMaxPipes * kPipeWords;
  c.g1_done = c.filled + max_mtiles * 4;
  c.g2_done = c.g1_done + max_mtiles;
  c.grp_first = c.g2_done + max_mtiles;
  c.grp_len = c.grp_first + max_mtiles;
  c.phase_start = c.grp_len + max_mtiles;
  c.slot_epoch = c.phase_start + 2 * max_mtiles + kMaxPipes;
  c.resident = c.slot_epoch + max_slots;
  c.words = c.resident + max_mtiles * 4;
  return c;
}

// pipeline p of n_part owns row tiles [lo, hi): a balanced contiguous split
MOE_HD void pipe_range(int n_mt, int n_part, int p, int* lo, int* hi) {
  *lo = int((long long)n_mt * p / n_part);
  *hi = int((long long)n_mt * (p + 1) / n_part);
}

// Group the row tiles [lo, hi) into runs of one expert, at most G row tiles each; an
// expert's run is split into the fewest such groups, of near-equal size (5 row tiles with
// G = 4 become 3 + 2, not 4 + 1: a group of one row tile reads its weight panels alone).
// expert_of(m) gives the local expert of row tile m.  Returns the number of groups.
template <class ExpertOf>
MOE_HD int build_groups(int lo, int hi, int G, ExpertOf expert_of, int* grp_first, int* grp_len) {
  int n = 0;
  int m = lo;
  while (m < hi) {
    const int e = expert_of(m);
    int run = 1;                                   // this expert's row tiles from m on
    while (m + run < hi && expert_of(m + run) == e) ++run;
    const int ng = (run + G - 1) / G;              // fewest groups of at most G row tiles,
    for (int i = 0; i < ng; ++i) {                 // sizes differing by at most one
      const int len = run / ng + (i < run % ng ? 1 : 0);
      grp_first[n] = m;
      grp_len[n] = len;
      ++n;
      m += len;
    }
  }
  return n;
}

// Phase k of 2n: down (1) or gate/up (0) tasks of group *g.
MOE_HD void phase_of(int k, int n, bool lookahead, int* down, int* g) {
  if (!lookahead) {
    *down = k & 1;
    *g = k >> 1;
    return;
  }
  if (k == 0) {
    *down = 0;
    *g = 0;
    return;
  }
  const int u = k - 1, gg = u >> 1;
  if (gg < n - 1) {
    *down = u & 1;
    *g = (u & 1) ? gg : gg + 1;
  } else {
    *down = 1;
    *g = n - 1;
  }
}

// Ticket prefix of the 2n phases (phase_start[2n] = tickets).  Returns the ticket count.
MOE_HD int build_phases(int n, const int* grp_len, int NT1, int NT2, bool lookahead, int* phase_start) {
  int t = 0;
  for (int k = 0; k < 2 * n; ++k) {
    int dn, g;
    phase_of(k, n, lookahead, &dn, &g);
    phase_start[k] = t;
    t += grp_len[g] * (dn ? NT2 : NT1);
  }
  phase_start[2 * n] = t;
  return t;
}

struct Task {
  int down;   // 0: gate/up tile, 1: down tile
  int m;      // row tile (global index)
  int j;      // column tile
};

// The task of ticket t (0 <= t < tickets) of a pipeline with n >= 1 groups.
MOE_HD Task task_of_ticket(int t, int n, const int* phase_start, const int* grp_first, const int* grp_len,
                           bool lookahead) {
  int lo = 0, hi = 2 * n - 1;                 // largest phase k with phase_start[k] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (phase_start[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  int dn, g;
  phase_of(lo, n, lookahead, &dn, &g);
  const int u = t - phase_start[lo], len = grp_len[g];
  Task r;
  r.down = dn;
  r.j = u / len;                              // panel-major: consecutive tickets share panel j
  r.m = grp_first[g] + (u - r.j * len);
  return r;
}

// ring slot (pipeline-local) of pipeline-local chunk q, and the epoch it must have reached
MOE_HD int chunk_slot(int q, int S) { return q % S; }
MOE_HD int chunk_epoch(int q, int S) { return q / S; }
// control word holding the epoch of the slot of pipeline p's chunk q (every reader and every
// writer of a slot epoch goes through this)
MOE_HD int slot_epoch_word(const CtrlLayout& cl, int p, int S, int q) { return cl.slot_epoch + p * S + chunk_slot(q, S); }

// Mover actions
enum MoverAct { kIdle = 0, kPush = 1, kGather = 2, kDone = 3 };

// One claim attempt of a data-movement workgroup (thread 0).  Pushes go first: they free
// ring slots.  The push of pipeline-local chunk c is claimable once every down tile of its
// row tile lo + c / cpm finished; a gather of chunk q once its slot's previous occupant was
// pushed.  Claims are CAS on the pipeline's in-order counters, so every chunk is gathered
// and pushed exactly once, in order.  With gather_only, only a gather is tried (a compute
// workgroup that waits for a chunk helps gathering instead of spinning).  Ops: ld(word) ->
// int (relaxed atomic load), cas(word, expected, desired) -> bool.
template <class Ops>
MOE_HD int mover_claim(Ops& ops, const CtrlLayout& cl, int p, int lo, int n_m, int cpm, int S, int NT2, int* arg,
                       bool gather_only = false) {
  const int pipe_base = cl.pipe0 + p * kPipeWords;
  const int n_chunks = n_m * cpm;
  const int ci = gather_only ? n_chunks : ops.ld(pipe_base + kPushNext);
  if (ci < n_chunks && ops.ld(cl.g2_done + lo + ci / cpm) >= NT2) {
    if (ops.cas(pipe_base + kPushNext, ci, ci + 1)) {
      *arg = ci;
      return kPush;
    }
    return kIdle;                             // lost the race: try again next round
  }
  const int qi = ops.ld(pipe_base + kGatherNext);
  if (qi < n_chunks && ops.ld(slot_epoch_word(cl, p, S, qi)) >= chunk_epoch(qi, S)) {
    if (ops.cas(pipe_base + kGatherNext, qi, qi + 1)) {
      *arg = qi;
      return kGather;
    }
    return kIdle;
  }
  if (ci >= n_chunks && qi >= n_chunks) return kDone;
  return kIdle;
}

// Work stealing at the end of a launch (outputs stored straight to recv, so a down tile
// leaves nothing in the ring that its own pipeline must copy).  A compute workgroup whose
// pipeline has handed out all its tickets takes tickets of another pipeline's last phase --
// the down tiles of that pipeline's last group -- while there are any.  The last group's
// gate/up tiles release their counters at agent scope, so the h rows a stolen down tile
// reads are visible from another XCD.  A stolen ticket is an ordinary ticket of its
// pipeline (claimed on the same counter), so every task still runs exactly once, and a
// down tile waits only for gate/up tiles with smaller tickets: stealing adds no wait.
// One attempt on pipeline v: the ticket, kStealWait if v's next ticket is not in its last
// phase yet (or the CAS lost a race), kStealDone if v has no ticket left.
constexpr int kStealWait = -1, kStealDone = -2;

template <class Ops>
MOE_HD int steal_claim(Ops& ops, const CtrlLayout& cl, int v, int last_phase_start, int n_tickets) {
  const int w = cl.pipe0 + v * kPipeWords + kTicketNext;
  const int t = ops.ld(w);
  if (t >= n_tickets) return kStealDone;
  if (t < last_phase_start) return kStealWait;
  return ops.cas(w, t, t + 1) ? t : kStealWait;
}

// ---------------------------------------------------------------------------- host plan
// Pipelines, ring partition and roles for one launch.
struct Plan {
  int n_part;      // pipelines
  int light;       // 1: one pipeline per XCD (L2-local hand-offs)
  int S;           // ring slots per pipeline
  int comm_pp;     // data-movement workgroups per pipeline
  int lookahead;   // ring holds two groups
  int G;           // row tiles per group, at most
  int ok;          // 0: the ring cannot hold one row tile, or no compute workgroup is left
};

// cus: workgroups of the grid (one per CU); eight_xcds: the grid spreads round-robin over
// eight XCDs; slots: ring slots available; cpm: chunks per row tile; comm: requested
// data-movement workgroups in total.
inline Plan plan_persistent(int cus, bool eight_xcds, long long slots, int cpm, int comm) {
  Plan P{};
  const int parts[4] = {8, 4, 2, 1};
  for (int i = 0; i < 4; ++i) {
    const int np = parts[i];
    if (np > 1 && !eight_xcds) continue;
    const long long S = slots / np;
    const int cpp = comm / np > 0 ? comm / np : 1;
    if (S >= 2LL * cpm && cpp < cus / np) {
      P.n_part = np;
      P.S = int(S > (1LL << 30) ? (1LL << 30) : S);
      P.comm_pp = cpp;
      P.lookahead = 1;
      break;
    }
  }
  if (!P.n_part) {                            // no look-ahead: one pipeline, one row tile of ring
    const int cpp = comm > 0 ? comm : 1;
    if (slots < cpm || cpp >= cus) return P;
    P.n_part = 1;
    P.S = int(slots > (1LL << 30) ? (1LL << 30) : slots);
    P.comm_pp = cpp;
    P.lookahead = 0;
  }
  P.light = (P.n_part == 8) ? 1 : 0;
  // Group size: with look-ahead the ring should hold three groups, so the gathers of group
  // g + 1 reuse the slots of group g - 2, pushed long before; else two (then the gathers of
  // g + 1 wait for the pushes of g - 1, whose down tiles run just before); without
  // look-ahead, one group.
  const int g = !P.lookahead ? P.S / cpm : (P.S >= 3 * cpm ? P.S / (3 * cpm) : P.S / (2 * cpm));
  P.G = g < 1 ? 1 : (g > kMaxGroup ? kMaxGroup : g);
  P.ok = 1;
  return P;
}

}  // namespace sched
}  // namespace moe
