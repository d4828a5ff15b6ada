#include "blob_file.h"

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cerrno>
#include <cstring>

namespace moe {

BlobFile::~BlobFile() { close(); }

void BlobFile::close() {
  if (fd_ >= 0) ::close(fd_);
  fd_ = -1;
  direct_ = false;
}

bool BlobFile::open(const std::string& path, uint64_t base, uint64_t need_bytes, bool want_direct,
                    std::string* err) {
  close();
  int fd = -1;
  bool direct = false;
  if (want_direct && base % kDirectAlign == 0) {
    fd = ::open(path.c_str(), O_RDONLY | O_DIRECT | O_CLOEXEC);
    direct = fd >= 0;
  }
  if (fd < 0) fd = ::open(path.c_str(), O_RDONLY | O_CLOEXEC);
  if (fd < 0) {
    *err = "cannot open " + path + ": " + std::strerror(errno);
    return false;
  }
  struct stat st {};
  if (::fstat(fd, &st) != 0) {
    *err = "cannot stat " + path + ": " + std::strerror(errno);
    ::close(fd);
    return false;
  }
  if ((uint64_t)st.st_size < base + need_bytes) {
    *err = path + " holds " + std::to_string((uint64_t)st.st_size) + " bytes, the blob needs " +
           std::to_string(base + need_bytes);
    ::close(fd);
    return false;
  }
  fd_ = fd;
  direct_ = direct;
  base_ = base;
  return true;
}

bool BlobFile::read(uint64_t off, void* dst, size_t bytes, std::string* err) const {
  uint8_t* p = static_cast<uint8_t*>(dst);
  uint64_t pos = base_ + off;
  size_t left = bytes;
  while (left > 0) {
    const ssize_t n = ::pread(fd_, p, left, (off_t)pos);
    if (n < 0) {
      if (errno == EINTR) continue;
      *err = std::string("pread failed: ") + std::strerror(errno);
      return false;
    }
    if (n == 0) {
      *err = "pread hit the end of the blob file";
      return false;
    }
    p += n;
    pos += (uint64_t)n;
    left -= (size_t)n;
  }
  return true;
}

ReadWorkers::ReadWorkers(int n_threads) {
  for (int i = 0; i < n_threads; ++i) threads_.emplace_back([this] { run(); });
}

ReadWorkers::~ReadWorkers() {
  {
    std::lock_guard<std::mutex> g(mu_);
    stop_ = true;
  }
  work_cv_.notify_all();
  for (auto& t : threads_) t.join();
}

void ReadWorkers::start(const BlobFile* file, const std::vector<uint64_t>& off, const std::vector<void*>& dst,
                        const std::vector<size_t>& bytes, const std::vector<void*>& bounce) {
  {
    std::lock_guard<std::mutex> g(mu_);
    file_ = file;
    items_.clear();
    queue_.clear();
    for (size_t i = 0; i < off.size(); ++i) {
      items_.push_back(Item{off[i], dst[i], bounce.empty() ? nullptr : bounce[i], bytes[i], 0, std::string()});
      queue_.push_back(i);
    }
  }
  work_cv_.notify_all();
}

bool ReadWorkers::wait(size_t i, std::string* err) {
  std::unique_lock<std::mutex> g(mu_);
  done_cv_.wait(g, [&] { return items_[i].state != 0; });
  if (items_[i].state == 2) {
    *err = items_[i].err;
    return false;
  }
  return true;
}

void ReadWorkers::drain() {
  std::unique_lock<std::mutex> g(mu_);
  done_cv_.wait(g, [&] {
    for (const Item& it : items_)
      if (it.state == 0) return false;
    return true;
  });
}

void ReadWorkers::run() {
  for (;;) {
    size_t i;
    uint64_t off;
    void* dst;
    void* bounce;
    size_t bytes;
    const BlobFile* file;
    {
      std::unique_lock<std::mutex> g(mu_);
      work_cv_.wait(g, [&] { return stop_ || !queue_.empty(); });
      if (stop_) return;
      i = queue_.front();
      queue_.pop_front();
      off = items_[i].off;
      dst = items_[i].dst;
      bounce = items_[i].bounce;
      bytes = items_[i].bytes;
      file = file_;
    }
    std::string err;
    bool ok;
    if (bounce) {
      ok = file->read(off, bounce, bytes, &err);
      if (ok) std::memcpy(dst, bounce, bytes);
    } else {
      ok = file->read(off, dst, bytes, &err);
    }
    {
      std::lock_guard<std::mutex> g(mu_);
      items_[i].state = ok ? 1 : 2;
      if (!ok) items_[i].err = err;
    }
    done_cv_.notify_all();
  }
}

}  // namespace moe
