// w4a4_resources.h — per-kernel resource figures of the compiled code objects
// (registers, LDS, spills), linked into the library as a table that the build
// generates from the code objects themselves, keyed by kernel symbol.
#pragma once

namespace w4a4 {

struct KernelResources {
  const char* symbol;   // mangled kernel name
  int vgpr, agpr, sgpr, lds, spill, scratch;
};

extern const KernelResources kKernelResources[];
extern const int kNumKernelResources;

}  // namespace w4a4
