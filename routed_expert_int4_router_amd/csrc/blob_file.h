// Storage-backed expert blob: the pool's miss path reading records from a
// file (host side, HIP-free).
//
// Pages: on a miss the runtime opens the repacked container read-only and
// issues one pread of the record bytes at blobBase + expertIndex *
// expertStride into a shared buffer (paotong.dev commentary, paragraph on the
// fetch path; alphalab.site field test, section on SSD reads, which also
// notes that a plain open() lets the OS page cache serve repeated reads and
// that bypassing it is a proposed follow-up). Here the file may be opened
// with O_DIRECT, the Linux counterpart of that bypass, and the reads run on a
// few worker threads so that the misses of one step are in flight together.
#pragma once

#include <condition_variable>
#include <cstddef>
#include <cstdint>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

namespace moe {

// Alignment O_DIRECT asks of buffers, offsets and lengths here.
constexpr uint64_t kDirectAlign = 4096;

class BlobFile {
 public:
  BlobFile() = default;
  BlobFile(const BlobFile&) = delete;
  BlobFile& operator=(const BlobFile&) = delete;
  ~BlobFile();

  // Opens `path` read-only. The file must hold at least base + need_bytes
  // bytes. With want_direct the page cache is bypassed (O_DIRECT) when the
  // filesystem supports it; otherwise, or without want_direct, reads are
  // buffered. Returns false with *err set on failure.
  bool open(const std::string& path, uint64_t base, uint64_t need_bytes, bool want_direct, std::string* err);
  void close();

  // Reads exactly `bytes` bytes at file offset base + off into dst, retrying
  // short reads. For a direct file, dst, base + off and bytes must be
  // multiples of kDirectAlign. Thread-safe (pread). Returns false with *err
  // set on an I/O error or end of file.
  bool read(uint64_t off, void* dst, size_t bytes, std::string* err) const;

  bool is_open() const { return fd_ >= 0; }
  bool direct() const { return direct_; }
  uint64_t base() const { return base_; }

 private:
  int fd_ = -1;
  bool direct_ = false;
  uint64_t base_ = 0;
};

// A fixed set of worker threads that run the reads of one batch; the caller
// waits for them one by one, in submission order.
class ReadWorkers {
 public:
  explicit ReadWorkers(int n_threads);
  ReadWorkers(const ReadWorkers&) = delete;
  ReadWorkers& operator=(const ReadWorkers&) = delete;
  ~ReadWorkers();

  // Starts a batch of reads from `file` (which must outlive the batch):
  // read i copies bytes[i] bytes at offset off[i] into dst[i]. When bounce is
  // non-empty, read i lands in bounce[i] first (ordinary, 4096-aligned
  // memory: direct I/O cannot target the driver's pinned mappings) and is
  // then copied to dst[i] by the same worker. Any earlier batch must have
  // been waited for completely.
  void start(const BlobFile* file, const std::vector<uint64_t>& off, const std::vector<void*>& dst,
             const std::vector<size_t>& bytes, const std::vector<void*>& bounce);
  // Blocks until read i of the current batch has finished; false with *err
  // set if it failed.
  bool wait(size_t i, std::string* err);
  // Blocks until every read of the current batch has finished (the caller
  // must do this, or wait for each read, before starting another batch).
  void drain();

 private:
  void run();

  struct Item {
    uint64_t off;
    void* dst;
    void* bounce;
    size_t bytes;
    int state;  // 0 queued or running, 1 done, 2 failed
    std::string err;
  };
  std::mutex mu_;
  std::condition_variable work_cv_, done_cv_;
  std::deque<size_t> queue_;
  std::vector<Item> items_;
  const BlobFile* file_ = nullptr;
  bool stop_ = false;
  std::vector<std::thread> threads_;
};

}  // namespace moe
