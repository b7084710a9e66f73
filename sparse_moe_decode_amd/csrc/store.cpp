// Storage tier under the pinned host pool: per-layer stacked bundle files
// read by byte range.
//
// Source: "The Other Half of the Memory Wall" §3.1 (expert weights stay on
// SSD as per-layer stacked files and are streamed on demand by byte range)
// and §5.3 (reads issued one token ahead move the load time off the critical
// path; the cost of a load grows with its cold bytes).
//
// Layer l's file holds its E expert bundles back to back (bundle e at byte
// e * bundle, the bundle layout of the staging path). A pool of I/O threads
// serves read requests: each bundle is one pread into a caller buffer
// (pinned host memory, so the GPU's staging copy reads it directly). With
// O_DIRECT the page cache is bypassed, so every read reaches the device;
// the driver's pinned pages cannot take a direct read, so each thread reads
// into its own page-aligned bounce buffer and copies the bundle over.
// Requests are grouped under tickets; e0_store_wait blocks until a ticket's
// reads are done and reports how long it blocked.

#include <fcntl.h>
#include <unistd.h>

#include <cerrno>

#include <chrono>
#include <condition_variable>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <unordered_map>
#include <vector>

#include "sparse_moe_decode.h"

int smd_report(int code, const char* msg);

namespace {

struct Req {
  int fd;
  int64_t off, bytes;
  char* dst;
  int64_t ticket;
};

struct Ticket {
  int pending = 0;
  int errors = 0;
  int first_errno = 0;  // errno of the first failed read (0: short read)
  double t_first = 0.0;  // issue time, seconds
  double t_done = 0.0;   // completion of the last read
};

double now_s() {
  return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

}  // namespace

struct e0_store {
  std::vector<int> fds;
  int32_t E = 0;
  int64_t bundle = 0;
  bool direct = false;
  std::mutex mu;
  std::condition_variable cv_work, cv_done;
  std::deque<Req> queue;
  std::unordered_map<int64_t, Ticket> tickets;
  int64_t next_ticket = 1;
  bool stop = false;
  std::vector<std::thread> workers;
  int64_t bytes_read = 0, reads = 0;

  void worker() {
    char* bounce = nullptr;  // direct reads: page-aligned staging for one bundle
    if (direct && posix_memalign(reinterpret_cast<void**>(&bounce), 4096, (size_t)bundle) != 0)
      bounce = nullptr;
    for (;;) {
      Req r;
      {
        std::unique_lock<std::mutex> lk(mu);
        cv_work.wait(lk, [&] { return stop || !queue.empty(); });
        if (queue.empty()) {  // stop requested and nothing left
          free(bounce);
          return;
        }
        r = queue.front();
        queue.pop_front();
      }
      int64_t done = 0;
      bool ok = !direct || bounce != nullptr;
      int err = ok ? 0 : ENOMEM;
      char* into = direct ? bounce : r.dst;
      while (ok && done < r.bytes) {
        const ssize_t n = pread(r.fd, into + done, (size_t)(r.bytes - done), (off_t)(r.off + done));
        if (n <= 0) {
          ok = false;
          err = n < 0 ? errno : 0;
          break;
        }
        done += n;
      }
      if (ok && direct) memcpy(r.dst, bounce, (size_t)r.bytes);
      {
        std::lock_guard<std::mutex> lk(mu);
        Ticket& tk = tickets[r.ticket];
        tk.pending -= 1;
        if (!ok && tk.errors++ == 0) tk.first_errno = err;
        tk.t_done = now_s();
        bytes_read += done;
        reads += 1;
      }
      cv_done.notify_all();
    }
  }
};

extern "C" {

int e0_store_open(const char* const* paths, int32_t n_layers, int32_t n_experts,
                  int64_t bundle_bytes, int32_t io_threads, int32_t direct, e0_store** out) {
  if (!paths || !out || n_layers < 1 || n_experts < 1 || bundle_bytes < 1 || io_threads < 1 ||
      io_threads > 256)
    return smd_report(E0_ERR_ARG, "e0_store_open: bad argument");
  if (direct && bundle_bytes % 4096)
    return smd_report(E0_ERR_ALIGN, "e0_store_open: O_DIRECT needs 4096-byte multiples");
  *out = nullptr;
  e0_store* s = new e0_store();
  s->E = n_experts;
  s->bundle = bundle_bytes;
  s->direct = direct != 0;
  for (int l = 0; l < n_layers; ++l) {
    const int fd = open(paths[l], O_RDONLY | (direct ? O_DIRECT : 0));
    if (fd < 0) {
      for (int f : s->fds) close(f);
      delete s;
      return smd_report(E0_ERR_IO, (std::string("e0_store_open: cannot open ") +
                                    (paths[l] ? paths[l] : "(null)") + ": " + strerror(errno))
                                       .c_str());
    }
    s->fds.push_back(fd);
  }
  for (int i = 0; i < io_threads; ++i) s->workers.emplace_back([s] { s->worker(); });
  *out = s;
  return E0_OK;
}

void e0_store_close(e0_store* s) {
  if (!s) return;
  {
    std::lock_guard<std::mutex> lk(s->mu);
    s->stop = true;
  }
  s->cv_work.notify_all();
  for (auto& w : s->workers) w.join();
  for (int f : s->fds) close(f);
  delete s;
}

int e0_store_read(e0_store* s, int32_t layer, const int32_t* ids, int32_t n, void* const* dst,
                  int64_t* ticket) {
  if (!s || !ticket || (n > 0 && (!ids || !dst)))
    return smd_report(E0_ERR_ARG, "e0_store_read: null argument");
  if (layer < 0 || layer >= (int32_t)s->fds.size())
    return smd_report(E0_ERR_ARG, "e0_store_read: layer out of range");
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= s->E) return smd_report(E0_ERR_RANGE, "e0_store_read: bad id");
    if (!dst[i]) return smd_report(E0_ERR_ARG, "e0_store_read: null destination");
  }
  {
    std::lock_guard<std::mutex> lk(s->mu);
    const int64_t tk = s->next_ticket++;
    Ticket& t = s->tickets[tk];
    t.pending = n;
    t.t_first = now_s();
    t.t_done = t.t_first;
    for (int i = 0; i < n; ++i)
      s->queue.push_back(Req{s->fds[layer], (int64_t)ids[i] * s->bundle, s->bundle,
                             (char*)dst[i], tk});
    *ticket = tk;
  }
  s->cv_work.notify_all();
  return E0_OK;
}

int e0_store_wait(e0_store* s, int64_t ticket, double* blocked_s, double* read_s) {
  if (!s) return smd_report(E0_ERR_ARG, "e0_store_wait: null store");
  const double t0 = now_s();
  std::unique_lock<std::mutex> lk(s->mu);
  if (s->tickets.find(ticket) == s->tickets.end())
    return smd_report(E0_ERR_STATE, "e0_store_wait: unknown ticket");
  // look the ticket up again after every wake-up: reads queued meanwhile may
  // have rehashed the table
  s->cv_done.wait(lk, [&] { return s->tickets.find(ticket)->second.pending == 0; });
  const auto it = s->tickets.find(ticket);
  const Ticket t = it->second;
  s->tickets.erase(it);
  lk.unlock();
  if (blocked_s) *blocked_s = now_s() - t0;
  if (read_s) *read_s = t.t_done - t.t_first;
  if (t.errors)
    return smd_report(E0_ERR_IO, (std::string("e0_store_wait: ") + std::to_string(t.errors) +
                                  " read(s) failed: " +
                                  (t.first_errno ? strerror(t.first_errno) : "short read"))
                                     .c_str());
  return E0_OK;
}

int64_t e0_store_bytes(e0_store* s) {
  if (!s) return -1;
  std::lock_guard<std::mutex> lk(s->mu);
  return s->bytes_read;
}

}  // extern "C"
