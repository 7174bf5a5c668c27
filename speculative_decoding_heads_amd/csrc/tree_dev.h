// The opaque tree handle: a host copy (for launch sizes) and a device copy
// (read by the kernels) of the same medusa_tree_host buffers.
#pragma once
#include "medusa.h"

struct medusa_tree {
  medusa_tree_host host;
  medusa_tree_host* dev;
};
